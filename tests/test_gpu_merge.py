"""GPU parity: e0_lora_merge_requant (a LoRA delta merged into an int4 g64
matrix and requantised) against the oracle (oracle/merge.py), which takes the
requantisation's definition in fp64. The kernel forms w' and the quotient
(w' - b') / s' in fp32, so its integer decisions may differ from the fp64
ones only where the fp64 value sits within the fp32 path's rounding error of
a flip. The check is exact everywhere else:

- scale and bias: the oracle's fp16 bits, except where (max - min) / 15 (or
  min) lies within EPS_SCALE (relative) of an fp16 rounding boundary; there
  one fp16 step either way is allowed;
- codes: clamp(round_half_even(u)) with u the fp64 quotient taken against the
  kernel's own scale and bias, except where u lies within EPS_CODE of a
  half-integer; there one code either way is allowed.

The fp32 path's error: s*q is exact in fp32, each B*A product of fp16 values
is exact, so w' carries at most r + 2 roundings of 2^-24 relative to terms
below 1 in size (|w'| < 0.4, |alpha B A| < 0.5 here), about 1e-6 absolute,
and the quotient two more roundings of a value below 16. Divided by the
smallest merged scale of these inputs (about 0.005) that is below 3e-4 code
units, under EPS_CODE = 2^-10; the range / 15 in fp32 is within 2^-21
relative of the fp64 one, under EPS_SCALE = 2^-16.

Covers the pages' delta magnitude (RMS about 1e-3) and a large one, ragged
shapes (one tile, a partial block of groups), rank 1 and 64, a zero delta,
constant groups, and an expert's gate and down matrices at full size."""
import numpy as np
import pytest

from e0inputs import gen
from oracle import merge as M
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _inputs(rows, cols, r, std, seed=21):
    q, s, b = gen.quant_matrix(gen.stream_key(seed, rows, cols, 1), gen.stream_key(seed, rows, cols, 2),
                               gen.stream_key(seed, rows, cols, 3), rows, cols)
    lb = gen.normal_f16(gen.stream_key(seed, rows, cols, 4), rows * r, std).view(np.uint16).reshape(rows, r)
    la = gen.normal_f16(gen.stream_key(seed, rows, cols, 5), r * cols, std).view(np.uint16).reshape(r, cols)
    return q, s, b, lb, la


def _gpu(q, s, b, lb, la, alpha):
    T = U.torch()
    rows, cols = q.shape[0], q.shape[1] * 8
    r = lb.shape[1]
    ngrp = cols // 64
    d = U.dev()
    t = lambda a, dt: T.from_numpy(np.ascontiguousarray(a).view(dt)).to(d)
    qd = t(q, np.int32)
    sd = t(gen._tile8(s).reshape(-1), np.int16)
    bd = t(gen._tile8(b).reshape(-1), np.int16)
    lbd, lad = t(lb, np.int16), t(la, np.int16)
    qo = T.empty_like(qd)
    so = T.empty((rows * ngrp,), dtype=T.int16, device=d)
    bo = T.empty_like(so)
    E().e0_lora_merge_requant(rows, cols, qd, sd, bd, lbd, lad, r, alpha, qo, so, bo)
    T.cuda.synchronize()
    return (qo.cpu().numpy().view(np.uint32),
            gen._untile8(so.cpu().numpy().view(np.uint16), rows, ngrp),
            gen._untile8(bo.cpu().numpy().view(np.uint16), rows, ngrp))


EPS_CODE = 2.0 ** -10
EPS_SCALE = 2.0 ** -16


def _fp16_steps(a, b):
    """Distance in fp16 steps between two arrays of fp16 bit patterns (same sign)."""
    a = a.view(np.int16).astype(np.int64)
    b = b.view(np.int16).astype(np.int64)
    key = lambda v: np.where(v < 0, -(v & 0x7FFF), v)  # sign-magnitude -> ordered integers
    return np.abs(key(a) - key(b))


def _check(q, s, b, lb, la, alpha=2.0):
    got = _gpu(q, s, b, lb, la, alpha)
    rows, cols = q.shape[0], q.shape[1] * 8
    w = M.merged_weights(q, s, b, lb, la, alpha)
    exact, s16, b16 = M.group_scale_bias(w)
    lo = w.reshape(rows, cols // 64, 64).min(axis=2)
    gs, gb = got[1], got[2]
    for name, g, e, v in (("scale", gs, s16.view(np.uint16), exact), ("bias", gb, b16.view(np.uint16), lo)):
        diff = g != e
        near = M.scale_boundary_distance(v) <= EPS_SCALE
        assert not np.any(diff & ~near), f"{name}: {int(np.sum(diff & ~near))} groups differ away from a boundary"
        assert np.all(_fp16_steps(g[diff], e[diff]) <= 1), f"{name}: a difference beyond one fp16 step"
    u = M.quotients(w, gs.view(np.float16), gb.view(np.float16))
    ref = M.codes_from_quotients(u)
    c = M.codes(got[0], cols)
    diff = c != ref
    near = M.boundary_distance(u) <= EPS_CODE
    assert not np.any(diff & ~near), f"codes: {int(np.sum(diff & ~near))} of {c.size} differ away from a half-integer"
    assert np.all(np.abs(c[diff].astype(np.int64) - ref[diff].astype(np.int64)) == 1)
    print(f"{rows}x{cols}: codes equal to the fp64 decision {c.size - int(diff.sum())} / {c.size} "
          f"({int(near.sum())} within {EPS_CODE:g} of a half-integer, {int(diff.sum())} of them differ); "
          f"scales differing {int((gs != s16.view(np.uint16)).sum())}, biases {int((gb != b16.view(np.uint16)).sum())}")
    # where no decision sits near a boundary, the whole matrix equals the oracle's
    if not np.any(near) and not np.any(M.scale_boundary_distance(exact) <= EPS_SCALE):
        ref_all = M.merge_requant(q, s, b, lb, la, alpha)
        assert all(np.array_equal(x, y) for x, y in zip(got, ref_all))
    return got


@pytest.mark.parametrize("rows,cols,r,std", [(64, 512, 16, 0.0112), (64, 512, 16, 0.112), (8, 64, 1, 0.05),
                                             (16, 64 * 40, 64, 0.01), (24, 192, 5, 0.3)])
def test_merge_matches_oracle(rows, cols, r, std):
    _check(*_inputs(rows, cols, r, std))


def test_zero_delta_and_constant_groups():
    q, s, b, lb, la = _inputs(32, 256, 8, 0.05)
    _check(q, s, b, np.zeros_like(lb), np.zeros_like(la))
    s0 = s.copy()
    s0[:, ::2] = 0  # every other group constant (scale 0): merged scale 0 where the delta is zero too
    got = _check(q, s0, b, np.zeros_like(lb), np.zeros_like(la))
    assert np.all(got[1][:, ::2] == 0)


@pytest.mark.parametrize("rows,cols", [(512, 2048), (2048, 512)])
def test_merge_full_expert_matrix(rows, cols):
    q, s, b, lb, la = _inputs(rows, cols, 16, 0.0112)
    got = _check(q, s, b, lb, la)
    ret = M.retention((q, s, b), got, lb, la, 2.0)
    print(f"{rows}x{cols} r=16 delta RMS ~1e-3: retention {ret:.3f}")
