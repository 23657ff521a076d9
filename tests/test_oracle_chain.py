"""Oracle pins for the chained batch-1 decode (norm -> staged MoE -> residual
over the stacked layers) and its fp16 rounding.

The rounding is pinned to Python's own binary16 packing (struct 'e', round to
nearest even). The chain is pinned by invariants that hold exactly (zero
routing weights or zero norm gain leave the residual untouched; a power-of-two
scale of the residual leaves the first layer's input unchanged) and by a
pure-Python brute force on a tiny stack."""
import math
import struct

import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W


def _py_half_bits(v: float) -> int:
    try:
        return struct.unpack("<H", struct.pack("<e", v))[0]
    except OverflowError:
        return 0x7C00 | (0x8000 if v < 0 else 0)


def test_to_half_matches_binary16_packing():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.normal(0, 1, 2000), rng.normal(0, 1e-5, 1000), rng.normal(0, 3e4, 500),
        np.ldexp(rng.integers(0, 2048, 500).astype(np.float64) + 0.5, -24),   # subnormal ties
        np.ldexp(rng.integers(1024, 2048, 500).astype(np.float64) + 0.5, -10),  # ties in [1, 2)
        np.array([0.0, -0.0, 65504.0, 65519.9, 65520.0, -65536.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -26,
                  2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -12), 1.0, -1.0, 1e-30])])
    got = oracle.to_half(vals)
    want = np.array([_py_half_bits(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(vals[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def _stack(cfg, L):
    """Pool = every expert of each layer in slot e (S = E)."""
    mats = [gen.expert(cfg.seed, l, e, cfg.d, cfg.f) for l in range(L) for e in range(cfg.E)]
    slot_of = np.tile(np.arange(cfg.E, dtype=np.int32), (L, 1))
    return mats, oracle.Experts(mats), slot_of


def _routing(cfg, L, step=0):
    lg = np.stack([W.given_logits(cfg, step, l)[0] for l in range(L)]).astype(np.float32)
    idx, w = oracle.softmax_topk(lg, cfg.K)
    return idx.astype(np.int32), w.astype(np.float64)


CFG = W.scaled(W.CHAIN35, d=128, f=64, E=6, K=2, L=3)


def test_zero_weights_or_zero_gain_leave_the_residual():
    L = CFG.L
    _, pool, slot_of = _stack(CFG, L)
    idx, w = _routing(CFG, L)
    r0 = W.residual0(CFG, 0).astype(np.float64)
    g = np.stack([W.norm_weight(CFG, l) for l in range(L)])
    y, r, err = oracle.chain_decode(pool, CFG.E, slot_of, CFG.E, CFG.d, CFG.f, r0, g, 1e-6, idx, np.zeros_like(w))
    assert err == 0 and not y.any() and all(np.array_equal(r[l], r0) for l in range(L))
    y, r, err = oracle.chain_decode(pool, CFG.E, slot_of, CFG.E, CFG.d, CFG.f, r0, np.zeros_like(g), 1e-6, idx, w)
    assert err == 0 and not y.any() and all(np.array_equal(r[l], r0) for l in range(L))
    y, r, err = oracle.chain_decode(pool, CFG.E, slot_of, CFG.E, CFG.d, CFG.f, r0, g, 1e-6, idx, w)
    assert err == 0 and np.abs(y).min(axis=1).max() > 0  # the real chain does move the residual


def test_first_layer_input_is_scale_invariant():
    L = CFG.L
    _, pool, slot_of = _stack(CFG, L)
    idx, w = _routing(CFG, L)
    r0 = W.residual0(CFG, 0).astype(np.float64)
    g = np.stack([W.norm_weight(CFG, l) for l in range(L)])
    y1, r1, _ = oracle.chain_decode(pool, CFG.E, slot_of, CFG.E, CFG.d, CFG.f, r0, g, 0.0, idx, w)
    y4, r4, _ = oracle.chain_decode(pool, CFG.E, slot_of, CFG.E, CFG.d, CFG.f, 4.0 * r0, g, 0.0, idx, w)
    assert np.array_equal(y1[0], y4[0])
    assert np.array_equal(r4[0], 4.0 * r0 + y1[0])


def _brute_chain(mats, E, d, f, slot_of, r0, g, eps, idx, w):
    """Pure-Python loops over a tiny stack; fp16 rounding by struct packing."""
    def half(bits):
        return struct.unpack("<e", struct.pack("<H", int(bits)))[0]

    def weight(m, rows, cols, r, c):
        q, s, b = m
        code = (int(q[r][c // 8]) >> (4 * (c % 8))) & 15
        return half(s[r][c // 64]) * code + half(b[r][c // 64])

    L, K = len(idx), len(idx[0])
    r = [float(v) for v in r0]
    ys, rs = [], []
    for l in range(L):
        inv = 1.0 / math.sqrt(sum(v * v for v in r) / d + eps)
        x = [half(_py_half_bits(r[i] * inv * half(g[l][i]))) for i in range(d)]
        y = [0.0] * d
        for k in range(K):
            gate, up, down = mats[l * E + int(slot_of[l][idx[l][k]])]
            h = []
            for j in range(f):
                a = sum(weight(gate, f, d, j, i) * x[i] for i in range(d))
                u = sum(weight(up, f, d, j, i) * x[i] for i in range(d))
                h.append(a / (1.0 + math.exp(-a)) * u)
            for i in range(d):
                y[i] += w[l][k] * sum(weight(down, d, f, i, j) * h[j] for j in range(f))
        r = [r[i] + y[i] for i in range(d)]
        ys.append(y)
        rs.append(list(r))
    return np.array(ys), np.array(rs)


def test_chain_matches_brute_force_on_a_tiny_stack():
    cfg = W.scaled(W.CHAIN35, d=64, f=64, E=4, K=2, L=2)
    mats, pool, slot_of = _stack(cfg, cfg.L)
    idx, w = _routing(cfg, cfg.L)
    r0 = W.residual0(cfg, 0).astype(np.float64)
    g = np.stack([W.norm_weight(cfg, l) for l in range(cfg.L)])
    y, r, err = oracle.chain_decode(pool, cfg.E, slot_of, cfg.E, cfg.d, cfg.f, r0, g, 1e-6, idx, w)
    yb, rb = _brute_chain(mats, cfg.E, cfg.d, cfg.f, slot_of, r0, g.view(np.uint16), 1e-6, idx, w)
    assert err == 0
    assert np.abs(y - yb).max() <= 1e-9 * np.abs(yb).max()
    assert np.abs(r - rb).max() <= 1e-9 * np.abs(rb).max()


def test_unresident_expert_is_flagged_and_skipped():
    L = 1
    _, pool, slot_of = _stack(CFG, L)
    idx, w = _routing(CFG, L)
    so = slot_of.copy()
    so[0, idx[0, 0]] = -1
    r0 = W.residual0(CFG, 0).astype(np.float64)
    g = W.norm_weight(CFG, 0)[None]
    y, _, err = oracle.chain_decode(pool, CFG.E, so, CFG.E, CFG.d, CFG.f, r0, g, 1e-6, idx, w)
    y1, _, _ = oracle.chain_decode(pool, CFG.E, slot_of, CFG.E, CFG.d, CFG.f, r0, g, 1e-6, idx[:, 1:], w[:, 1:])
    assert err == 2 and np.array_equal(y, y1)
