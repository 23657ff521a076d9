"""Helpers for the GPU parity tests: device buffers from generated inputs."""
from __future__ import annotations

import numpy as np

from e0inputs import gen


def torch():
    import torch as T
    return T


def dev():
    return torch().device("cuda:0")


def f16(a: np.ndarray):
    """fp16 numpy array -> int16 device tensor with the same bits."""
    return torch().from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev())


def i32(a):
    return torch().from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(dev())


def f32(a):
    return torch().from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to(dev())


def empty(shape, dtype="float32"):
    T = torch()
    return T.empty(shape, dtype=getattr(T, dtype), device=dev())


def zeros(shape, dtype="float32"):
    T = torch()
    return T.zeros(shape, dtype=getattr(T, dtype), device=dev())


def full(shape, v, dtype="int32"):
    T = torch()
    return T.full(shape, v, dtype=getattr(T, dtype), device=dev())


def gpu_store(cfg, layers, tag=gen.TAG_EXPERT):
    """uint8 [len(layers)][E][bundle] device tensor filled on the GPU."""
    from e0inputs import gpu as G
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    st = zeros((len(layers), cfg.E, bb), "uint8")
    for i, l in enumerate(layers):
        G.fill_experts(st[i].data_ptr(), bb, cfg.seed, l, range(cfg.E), cfg.d, cfg.f, tag)
    return st


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def bytes_of(t):
    return t.numel() * t.element_size()


def elem_err(got, ref) -> float:
    """Largest per-row ratio max_i |got - ref| / max_i |ref| (rows = last axis)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g2 = got.reshape(-1, got.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    num = np.max(np.abs(g2 - r2), axis=1)
    den = np.maximum(np.max(np.abs(r2), axis=1), 1e-300)
    return float(np.max(num / den))


def assert_close(got, ref, rel_l2_tol: float, elem_tol: float, what: str = ""):
    """Both bars: whole-array rel-L2 and, per row, the largest element error
    against the row's largest reference value (a sparse indexing mistake that
    the norm would average away fails the second). Returns (rel_l2, elem)."""
    r, e = rel_l2(got, ref), elem_err(got, ref)
    assert r <= rel_l2_tol and e <= elem_tol, (what, r, e)
    return r, e
