"""Build libe0.so (the gfx950 HIP kernels behind include/e0.h) in-tree with hipcc.

Every source is compiled to an object in parallel (each is its own
translation unit with its own device code), then the objects are linked."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libe0.so")
SOURCES = ["api.hip", "route.hip", "decode.hip", "slot.hip", "prerouter.hip", "prefill.hip", "merge.hip",
           "noalloc.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-gpu-flush-denormals-to-zero"]
# decode.hip: the batched down kernel's matrix-core products are scaled and
# summed by ordinary vector instructions right after each MFMA; in VGPRs they
# need no AccVGPR copies (32 fewer instructions per pass).
SOURCE_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in r.stderr.splitlines() if NOISE not in ln)
    return r.returncode, err


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ, s.replace(".hip", ".o"))
        jobs.append((obj, [HIPCC, *FLAGS, *SOURCE_FLAGS.get(s, ()), *extra, "-c", os.path.join(CSRC, s), "-o", obj]))
    if verbose:
        for _, cmd in jobs:
            print(" ".join(cmd), flush=True)
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 1)) as ex:
        res = list(ex.map(lambda j: _run(j[1]), jobs))
    for (obj, _), (rc, err) in zip(jobs, res):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(obj)} ({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    rc, err = _run(link)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
