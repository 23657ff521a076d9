"""Pins of the merged-LoRA oracle (oracle/merge.py) against what the format
and the arithmetic fix, independent of its own code:
- requantising a group that already lies on a 16-level grid (zero delta)
  gives back its codes, scale and bias exactly (the scale rule is range / 15,
  not / 16);
- quotients that fall exactly on a half-integer round to the even code;
- a constant group has scale 0, codes 0 and its value as bias;
- the group's least value takes code 0 and its largest code 15;
- every requantised weight is within half a step (plus the fp16 rounding of
  scale and bias) of the merged fp32 weight;
- the merged weights (rank sum written term by term) agree with base +
  alpha * B @ A from numpy's matrix product (a transposed or mis-indexed
  operand fails);
- the boundary helpers a GPU parity check uses give the distances of known
  points to the nearest rounding flip;
- retention (jaehun.me review, the paragraph on not merging; xyznot.com FAQ on
  the unmerged recovery LoRA): a delta far below one 4-bit step is mostly
  erased, one far above it mostly kept, an exact whole-step shift kept."""
import numpy as np

from e0inputs import gen
from oracle import merge as M


def _base(rows, cols, seed=7):
    return gen.quant_matrix(gen.stream_key(seed, 1), gen.stream_key(seed, 2), gen.stream_key(seed, 3), rows, cols)


def _lora(rows, cols, r, std, seed=11):
    b = gen.normal_f16(gen.stream_key(seed, 4), rows * r, std).reshape(rows, r)
    a = gen.normal_f16(gen.stream_key(seed, 5), r * cols, std).reshape(r, cols)
    return b.view(np.uint16), a.view(np.uint16)


def test_zero_delta_on_full_grid_keeps_codes():
    rows, cols = 16, 128
    q, s, b = _base(rows, cols)
    c = M.codes(q, cols).reshape(rows, cols // 64, 64)
    c[:, :, 0] = 0   # every group spans the whole grid 0 .. 15
    c[:, :, 1] = 15
    q = M.pack(c.reshape(rows, cols))
    zb = np.zeros((rows, 4), dtype=np.uint16)
    za = np.zeros((4, cols), dtype=np.uint16)
    q2, s2, b2 = M.merge_requant(q, s, b, zb, za, 2.0)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2, s)  # 15 s / 15 = s exactly in fp64
    assert np.array_equal(b2, b)


def test_constant_group_has_zero_scale():
    rows, cols = 8, 64
    q = np.zeros((rows, cols // 8), dtype=np.uint32)
    s = np.full((rows, 1), np.float16(0.01).view(np.uint16), dtype=np.uint16)
    b = np.full((rows, 1), np.float16(-0.03125).view(np.uint16), dtype=np.uint16)
    zb = np.zeros((rows, 2), dtype=np.uint16)
    za = np.zeros((2, cols), dtype=np.uint16)
    q2, s2, b2 = M.merge_requant(q, s, b, zb, za, 2.0)
    assert np.all(q2 == 0) and np.all(s2 == 0)
    assert np.all(b2.view(np.float16) == np.float16(-0.03125))


def test_extremes_take_codes_0_and_15_and_error_within_half_step():
    rows, cols, r = 32, 256, 8
    q, s, b = _base(rows, cols)
    lb, la = _lora(rows, cols, r, 0.05)
    w = M.merged_weights(q, s, b, lb, la, 2.0)
    q2, s2, b2 = M.requantize(w)
    c = M.codes(q2, cols).reshape(rows, cols // 64, 64)
    g = w.reshape(rows, cols // 64, 64)
    assert np.all(c[np.arange(rows)[:, None], np.arange(cols // 64)[None, :], g.argmin(axis=2)] == 0)
    assert np.all(c[np.arange(rows)[:, None], np.arange(cols // 64)[None, :], g.argmax(axis=2)] == 15)
    deq = M.dequant64(q2, s2, b2).reshape(rows, cols // 64, 64)
    s16 = s2.view(np.float16).astype(np.float64)[:, :, None]
    lo = g.min(axis=2).astype(np.float64)[:, :, None]
    hi = g.max(axis=2).astype(np.float64)[:, :, None]
    slack = np.abs(b2.view(np.float16).astype(np.float64)[:, :, None] - lo) + 15 * np.abs(s16 - (hi - lo) / 15)
    assert np.all(np.abs(deq - g) <= 0.5 * s16 + slack + 1e-7)


def test_merged_weights_match_fp64_matrix_product():
    rows, cols, r = 24, 192, 5
    q, s, b = _base(rows, cols)
    lb, la = _lora(rows, cols, r, 0.1)
    w = M.merged_weights(q, s, b, lb, la, 2.0)
    ref = M.dequant64(q, s, b) + 2.0 * (lb.view(np.float16).astype(np.float64) @ la.view(np.float16).astype(np.float64))
    assert np.max(np.abs(w - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))
    # a transposed operand (B^T-shaped use of A) is caught
    bad = M.dequant64(q, s, b) + 2.0 * (lb.view(np.float16).astype(np.float64)
                                        @ np.roll(la.view(np.float16).astype(np.float64), 1, axis=1))
    assert np.max(np.abs(w - bad)) > 1e-3


def test_retention_small_delta_erased_large_delta_kept():
    rows, cols, r = 64, 512, 16
    base = _base(rows, cols)
    small = _lora(rows, cols, r, 0.0112)   # alpha * B A has RMS about 1e-3 (the pages' magnitude)
    large = _lora(rows, cols, r, 0.56)     # RMS about 2.6, far above one step (0.005 .. 0.02)
    rs = M.retention(base, M.merge_requant(*base, *small, 2.0), *small, 2.0)
    rl = M.retention(base, M.merge_requant(*base, *large, 2.0), *large, 2.0)
    assert rs < 0.5, rs
    assert rl > 0.9, rl


def test_retention_of_whole_step_shift_is_one():
    # alpha B A = a constant equal to one grid step, on groups whose codes span
    # 0 .. 15: the merged grid is the old one shifted by a step, exactly (same
    # scale, bias + step, same codes), so nothing of the delta is lost.
    rows, cols = 8, 64
    c = np.tile(np.arange(64) % 16, (rows, 1))
    q = M.pack(c)
    s = np.full((rows, 1), np.float16(0.015625).view(np.uint16), dtype=np.uint16)   # 2^-6
    b = np.full((rows, 1), np.float16(-0.125).view(np.uint16), dtype=np.uint16)
    lb = np.full((rows, 1), np.float16(0.125).view(np.uint16), dtype=np.uint16)
    la = np.full((1, cols), np.float16(0.0625).view(np.uint16), dtype=np.uint16)   # alpha * 0.125 * 0.0625 = 2^-6
    merged = M.merge_requant(q, s, b, lb, la, 2.0)
    assert np.array_equal(merged[0], q) and np.array_equal(merged[1], s)
    assert np.all(merged[2].view(np.float16) == np.float16(-0.125 + 0.015625))
    assert abs(M.retention((q, s, b), merged, lb, la, 2.0) - 1.0) < 1e-12


def test_half_integer_quotients_round_to_even():
    # One group, scale 2^-6 and bias 0 exactly (least 0, largest 15 * 2^-6), the
    # other weights placed so that (w - b) / s is k + 1/2 exactly for k = 0..13:
    # round half to even gives 0, 2, 2, 4, 4, ..., 14 (a half-up rule would give
    # 1, 2, 3, ...; a truncation 0, 1, 2, ...).
    step = 2.0 ** -6
    w = np.zeros((1, 64))
    w[0, 1] = 15 * step
    halves = np.arange(14) + 0.5
    w[0, 2:16] = halves * step
    w[0, 16:] = 7 * step
    q, s, b = M.requantize(w)
    assert s.view(np.float16)[0, 0] == np.float16(step) and b.view(np.float16)[0, 0] == 0
    c = M.codes(q, 64)[0]
    assert c[0] == 0 and c[1] == 15 and np.all(c[16:] == 7)
    assert c[2:16].tolist() == [0, 2, 2, 4, 4, 6, 6, 8, 8, 10, 10, 12, 12, 14]


def test_boundary_helpers_on_known_points():
    u = np.array([[0.5, 2.25, 3.0, 14.4999, np.nan]])
    d = M.boundary_distance(u)
    assert d[0, 0] == 0.0 and d[0, 1] == 0.25 and d[0, 2] == 0.5
    assert abs(d[0, 3] - 1e-4) < 1e-12 and np.isinf(d[0, 4])
    # fp16 values 1 and 1 + 2^-10: their midpoint 1 + 2^-11 is where rounding flips
    one = 1.0
    mid = 1.0 + 2.0 ** -11
    e = np.array([one, mid, mid * (1 + 1e-6), 0.0])
    sd = M.scale_boundary_distance(e)
    assert abs(sd[0] - 2.0 ** -11) < 1e-15
    assert sd[1] == 0.0
    assert abs(sd[2] - 1e-6) < 1e-9 and np.isinf(sd[3])
