"""GPU fill of expert stores with the generator of ``gen`` (bit-identical).

Input generation only. Keys are derived here on the host with ``gen.stream_key``;
e0inputs/csrc/fill.hip turns them into bundles on the GPU.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

from . import gen

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libe0gen.so")
_LIB = None


def build(verbose: bool = False) -> str:
    cmd = ["/opt/rocm/bin/hipcc", "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "csrc", "fill.hip"), "-o", LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not built")
        import torch  # noqa: F401  (bind to torch's HIP runtime, as in the libe0 binding)
        _LIB = C.CDLL(LIB_PATH)
        _LIB.e0gen_fill_experts.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                            C.c_void_p]
        _LIB.e0gen_fill_experts.restype = C.c_int
    return _LIB


def expert_keys(seed: int, layer: int, experts, tag: int = gen.TAG_EXPERT) -> np.ndarray:
    keys = np.empty((len(experts), 9), dtype=np.uint64)
    for i, e in enumerate(experts):
        for m in range(3):
            for p in range(3):
                keys[i, 3 * m + p] = gen.stream_key(seed, tag, layer, int(e), m, p)
    return keys


def fill_experts(dst_ptr: int, stride: int, seed: int, layer: int, experts, d: int, f: int,
                 tag: int = gen.TAG_EXPERT, stream=None):
    """Write the bundles of `experts` (ids) of `layer` at dst_ptr + i * stride."""
    import torch
    keys = torch.from_numpy(expert_keys(seed, layer, experts, tag).view(np.int64)).cuda()
    st = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = lib().e0gen_fill_experts(C.c_void_p(dst_ptr), stride, C.c_void_p(keys.data_ptr()), len(experts), d, f,
                                  C.c_void_p(st))
    if rc:
        raise RuntimeError(f"e0gen_fill_experts failed ({rc}" + (f": HIP error {rc - 1000}" if rc >= 1000 else "") + ")")
    torch.cuda.synchronize()  # keys must outlive the fill; this is set-up, not a timed path
    del keys
