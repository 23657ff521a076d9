"""Build the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: the product library never links or loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-fno-fast-math",
           "-ffp-contract=off", "-pthread", os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer, linked
    into the driver sanitize_check.c (a CPU executable; no GPU code)."""
    exe = os.path.join(HERE, "sanitize_check")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fno-fast-math", "-ffp-contract=off", "-pthread",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(HERE, "oracle.c"), os.path.join(HERE, "sanitize_check.c"), "-o", exe, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return exe


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
