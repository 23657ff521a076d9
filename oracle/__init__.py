"""ctypes face of the CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg. The GPU library and its Python binding never
import this package, and this package imports nothing of theirs.

All arrays are numpy; fp16 tensors are passed as float16 arrays (their bit
patterns), int4 matrices as (q uint32, s uint16, b uint16) triples.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class _Mat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("b", C.c_void_p)]


class _Expert(C.Structure):
    _fields_ = [("gate", _Mat), ("up", _Mat), ("down", _Mat)]


class _Lora(C.Structure):
    _fields_ = [("a", C.c_void_p), ("b", C.c_void_p)]


class _Head(C.Structure):
    _fields_ = [("fc1_w", C.c_void_p), ("fc1_b", C.c_void_p), ("fc2_w", C.c_void_p),
                ("fc2_b", C.c_void_p), ("lin_w", C.c_void_p)]


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build
            build.build()
        _LIB = C.CDLL(path)
        _LIB.orc_half.restype = C.c_double
        _LIB.orc_half.argtypes = [C.c_uint16]
        _LIB.orc_softmax_topk_margin.restype = C.c_double
        _LIB.orc_sigmoid_group_margin.restype = C.c_double
        _LIB.orc_to_half.restype = C.c_uint16
        _LIB.orc_to_half.argtypes = [C.c_double]
    return _LIB


def _p(a):
    return C.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Experts:
    """A list of experts (each [(q,s,b)] * 3) laid out as an orc_expert array.
    Holds references to the numpy arrays."""

    def __init__(self, mats_list):
        self.keep = []
        self.arr = (_Expert * max(1, len(mats_list)))()
        for i, mats in enumerate(mats_list):
            ms = []
            for (q, s, b) in mats:
                q = _c(q, np.uint32)
                s = _c(np.asarray(s).view(np.uint16), np.uint16)
                b = _c(np.asarray(b).view(np.uint16), np.uint16)
                self.keep += [q, s, b]
                ms.append(_Mat(q.ctypes.data, s.ctypes.data, b.ctypes.data))
            self.arr[i] = _Expert(*ms)
        self.n = len(mats_list)

    @property
    def ptr(self):
        return C.cast(self.arr, C.c_void_p)


def half(bits: int) -> float:
    return lib().orc_half(bits)


def dequant(q, s, b, rows, cols):
    q, s, b = _c(q, np.uint32), _c(np.asarray(s).view(np.uint16), np.uint16), _c(np.asarray(b).view(np.uint16), np.uint16)
    m = _Mat(q.ctypes.data, s.ctypes.data, b.ctypes.data)
    out = np.empty((rows, cols), dtype=np.float64)
    lib().orc_dequant(C.byref(m), rows, cols, _p(out))
    return out


def router_logits(x, wr):
    x = _c(x, np.float16)
    wr = _c(wr, np.float16)
    T, d = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(_p(x), _p(wr), T, E, d, _p(out))
    return out


def softmax_topk(logits, K):
    lg = _c(logits, np.float32)
    T, E = lg.shape
    idx = np.empty((T, K), dtype=np.int32)
    w = np.empty((T, K), dtype=np.float64)
    lib().orc_softmax_topk(_p(lg), T, E, K, _p(idx), _p(w))
    return idx, w


def sigmoid_group(logits, K, n_groups, topk_groups, scale, eps=1e-20):
    lg = _c(logits, np.float32)
    T, E = lg.shape
    idx = np.empty((T, K), dtype=np.int32)
    w = np.empty((T, K), dtype=np.float64)
    rc = lib().orc_sigmoid_group(_p(lg), T, E, K, n_groups, topk_groups, C.c_double(scale), C.c_double(eps),
                                 _p(idx), _p(w))
    if rc:
        raise ValueError("sigmoid_group: unsupported shape")
    return idx, w


def route(logits, cfg):
    """Route with the mode of a workload config."""
    if cfg.mode == 0:
        return softmax_topk(logits, cfg.K)
    return sigmoid_group(logits, cfg.K, cfg.n_groups, cfg.topk_groups, cfg.scale, cfg.eps)


def route_margin(logits, cfg) -> float:
    lg = _c(logits, np.float32)
    T, E = lg.shape
    if cfg.mode == 0:
        return lib().orc_softmax_topk_margin(_p(lg), T, E, cfg.K)
    return lib().orc_sigmoid_group_margin(_p(lg), T, E, cfg.K, cfg.n_groups, cfg.topk_groups)


def expert_ffn(mats, x, d, f):
    ex = Experts([mats])
    x = _c(x, np.float16)
    y = np.empty(d, dtype=np.float64)
    lib().orc_expert_ffn(ex.ptr, d, f, _p(x), _p(y))
    return y


def moe_exact(experts: Experts, d, f, x, idx, w):
    x, idx, w = _c(x, np.float16), _c(idx, np.int32), _c(w, np.float64)
    T, K = idx.shape
    y = np.empty((T, d), dtype=np.float64)
    err = lib().orc_moe_exact(experts.ptr, experts.n, d, f, T, K, _p(x), _p(idx), _p(w), _p(y))
    return y, err


def moe_staged(pool: Experts, slot_of, E, d, f, x, idx, w):
    x, idx, w, so = _c(x, np.float16), _c(idx, np.int32), _c(w, np.float64), _c(slot_of, np.int32)
    T, K = idx.shape
    y = np.empty((T, d), dtype=np.float64)
    err = lib().orc_moe_staged(pool.ptr, pool.n, _p(so), E, d, f, T, K, _p(x), _p(idx), _p(w), _p(y))
    return y, err


def moe_sorted(experts: Experts, d, f, x, idx, w):
    x, idx, w = _c(x, np.float16), _c(idx, np.int32), _c(w, np.float64)
    T, K = idx.shape
    y = np.empty((T, d), dtype=np.float64)
    perm = np.full(T * K, -1, dtype=np.int32)
    err = lib().orc_moe_sorted(experts.ptr, experts.n, d, f, T, K, _p(x), _p(idx), _p(w), _p(y), _p(perm))
    return y, err, perm


def slot_update(E, S, want, keep, slot_of, expert_of):
    """Returns (status, copies [(slot, expert)]); slot_of/expert_of updated in place."""
    want = _c(np.asarray(want).ravel(), np.int32)
    keep = _c(np.asarray(keep).ravel(), np.int32)
    assert slot_of.dtype == np.int32 and expert_of.dtype == np.int32
    assert slot_of.flags.c_contiguous and expert_of.flags.c_contiguous
    cs = np.empty(max(1, E), dtype=np.int32)
    ce = np.empty(max(1, E), dtype=np.int32)
    n = C.c_int32(0)
    rc = lib().orc_slot_update(E, S, _p(want), int(want.size), _p(keep), int(keep.size), _p(slot_of),
                               _p(expert_of), _p(cs), _p(ce), C.byref(n))
    return rc, list(zip(cs[:n.value].tolist(), ce[:n.value].tolist()))


def head_feature(h, E, cur, prev, K):
    h = _c(h, np.float16)
    d = h.size
    cur = _c(cur, np.int32)
    prev = None if prev is None else _c(prev, np.int32)
    out = np.empty(d + 2 * E, dtype=np.float64)
    lib().orc_head_feature(_p(h), d, E, _p(cur), _p(prev) if prev is not None else None, K, _p(out))
    return out


def _head_struct(hd):
    arrs = [_c(hd.fc1_w, np.float16), None if hd.fc1_b is None else _c(hd.fc1_b, np.float16),
            _c(hd.fc2_w, np.float16), None if hd.fc2_b is None else _c(hd.fc2_b, np.float16),
            _c(hd.lin_w, np.float16)]
    st = _Head(*[a.ctypes.data if a is not None else None for a in arrs])
    return st, arrs


def head_logits(hd, h, cur, prev, K):
    st, keep = _head_struct(hd)
    h = _c(h, np.float16)
    d = h.size
    E, hid = hd.fc2_w.shape
    cur = _c(cur, np.int32)
    prev = None if prev is None else _c(prev, np.int32)
    o = np.empty(E, dtype=np.float64)
    lib().orc_head_logits(C.byref(st), d, E, hid, _p(h), _p(cur), _p(prev) if prev is not None else None, K, _p(o))
    del keep
    return o


def shared_lora(mats, lora, r, alpha_over_r, x, d, f):
    ex = Experts([mats])
    x = _c(x, np.float16)
    y = np.empty(d, dtype=np.float64)
    if lora is None:
        lib().orc_shared_lora(ex.ptr, None, r, C.c_double(alpha_over_r), d, f, _p(x), _p(y))
    else:
        keep = [(_c(a, np.float16), _c(b, np.float16)) for (a, b) in lora]
        arr = (_Lora * 3)(*[_Lora(a.ctypes.data, b.ctypes.data) for (a, b) in keep])
        lib().orc_shared_lora(ex.ptr, arr, r, C.c_double(alpha_over_r), d, f, _p(x), _p(y))
    return y


def decode_layers(pools: Experts, S, slot_of, E, d, f, x, idx, w, n_threads=1):
    """pools: Experts of L*S entries (layer-major); slot_of [L,E]; x [L,B,d];
    idx, w [L,B,K] -> y [L,B,d]."""
    x, idx, w, so = _c(x, np.float16), _c(idx, np.int32), _c(w, np.float64), _c(slot_of, np.int32)
    L, B, K = idx.shape
    y = np.empty((L, B, d), dtype=np.float64)
    err = lib().orc_decode_layers(pools.ptr, S, _p(so), L, E, d, f, B, K, _p(x), _p(idx), _p(w), _p(y),
                                  n_threads)
    return y, err


def to_half(v):
    """Nearest binary16 bit patterns (ties to even) of float64 values."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    f = lib().orc_to_half
    return np.array([f(C.c_double(float(t))) for t in v.ravel()], dtype=np.uint16).reshape(v.shape)


def chain_decode(pools: Experts, S, slot_of, E, d, f, r0, g, eps, idx, w):
    """Chained batch-1 decode: pools Experts of L*S entries (layer-major),
    slot_of [L,E], r0 [d] (fp64), g fp16 [L,d], idx/w [L,K] ->
    (y [L,d], r_out [L,d]) with r_out[l] the residual after layer l."""
    so, idx, w = _c(slot_of, np.int32), _c(idx, np.int32), _c(w, np.float64)
    r0, g = _c(r0, np.float64), _c(g, np.float16)
    L, K = idx.shape
    y = np.empty((L, d), dtype=np.float64)
    r_out = np.empty((L, d), dtype=np.float64)
    err = lib().orc_chain_decode(pools.ptr, S, _p(so), L, E, d, f, K, _p(r0), _p(g), C.c_double(eps), _p(idx),
                                 _p(w), _p(y), _p(r_out))
    return y, r_out, err


def moe_by_expert(expert_fn, E, d, f, x, idx, w):
    """One MoE layer over T tokens with each active expert dequantised once
    (orc_dequant, fp64) and applied to all of its tokens as fp64 matrix
    products (numpy): the exact ordering of the combine (jaehun.me review,
    report 3.1, the whole-layer path) at sizes where the per-(token, k) C loop
    is too slow.

    expert_fn(e) -> [(q, s, b)] * 3 (gate [f][d], up [f][d], down [d][f]);
    x fp16 [T][d]; idx int32 [T][K]; w [T][K]. Pairs with an id outside
    0..E-1 contribute nothing. y [T][d] fp64 = sum over k, in k order, of
    w[t][k] * down(silu(gate x_t) * up x_t)."""
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    T, K = idx.shape
    yk = np.zeros((T, K, d), dtype=np.float64)
    for e in np.unique(idx):
        if e < 0 or e >= E:
            continue
        (gq, gs, gb), (uq, us, ub), (dq, ds, db) = expert_fn(int(e))
        G = dequant(gq, gs, gb, f, d)
        Uw = dequant(uq, us, ub, f, d)
        D = dequant(dq, ds, db, d, f)
        t, k = np.nonzero(idx == e)
        X = x64[t]
        a = X @ G.T
        h = a / (1.0 + np.exp(-a)) * (X @ Uw.T)
        yk[t, k] = w[t, k][:, None] * (h @ D.T)
    y = yk[:, 0].copy()
    for k in range(1, K):
        y += yk[:, k]
    return y
