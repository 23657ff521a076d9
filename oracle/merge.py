"""Oracle of the merged-LoRA alternative: a low-rank delta added to an int4
group-64 matrix and requantised, and the retention measure the pages use to
compare it with the unmerged delta.

TEST INFRASTRUCTURE ONLY: imported by tests/ and by the benchmark's
CPU-baseline leg, never by the GPU library or its binding.

Sources: jaehun.me review, the paragraph on not merging (citing the report's
section 3.3): retention = 1 - |U - M| / |U - B| with U the unmerged, M the
merged and B the base weights; xyznot.com FAQ on why the recovery LoRA stays
unmerged: deltas of RMS about 1e-3 sit below one 4-bit step, so merging and
requantising erases most of them. The pages do not print the requantisation
rule; this follows the plainest reading of the stacks' affine format, written
out from its definition in fp64:

    w'  = s*q + b + alpha * sum_k B[i,k] * A[k,c]           (fp64)
    s'  = fp16((max w' - min w') / 15)    per (row, 64-column group)
    b'  = fp16(min w')
    q'  = clamp(round_half_even((w' - b') / s'), 0, 15)     (0 where s' = 0)

s*q + b and every B*A product of fp16 values are exact in fp64; the quotient
is taken in fp64 against the fp16-rounded s' and b'. A GPU that computes w'
and the quotient in fp32 takes the same integer decision except where the
fp64 quotient lies within its rounding error of a half-integer, and the same
fp16 scale except where (max - min) / 15 lies that close to an fp16 rounding
boundary: ``boundary_distance`` and ``scale_boundary_distance`` give what a
parity check needs to allow exactly those cases.

Matrices are (q uint32 [rows][cols/8], s uint16 [rows][cols/64], b uint16
[rows][cols/64]) with fp16 bit patterns in s and b (the oracle's format);
lora_b is fp16 [rows][r], lora_a fp16 [r][cols].
"""
from __future__ import annotations

import numpy as np

GROUP = 64


def codes(q: np.ndarray, cols: int) -> np.ndarray:
    """uint32 words [rows][cols/8] -> codes [rows][cols] (code c at bits 4*(c%8) of word c/8)."""
    q = np.asarray(q, dtype=np.uint32)
    sh = (np.arange(8, dtype=np.uint32) * 4)[None, None, :]
    return ((q[:, :, None] >> sh) & np.uint32(15)).reshape(q.shape[0], cols)


def pack(c: np.ndarray) -> np.ndarray:
    """codes [rows][cols] (0..15) -> uint32 words [rows][cols/8]."""
    rows, cols = c.shape
    c = c.astype(np.uint32).reshape(rows, cols // 8, 8)
    return np.bitwise_or.reduce(c << (np.arange(8, dtype=np.uint32) * 4)[None, None, :], axis=2).astype(np.uint32)


def _f16(a) -> np.ndarray:
    return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant64(q, s, b) -> np.ndarray:
    """s*q + b in fp64 (exact for fp16 s, b and 4-bit q)."""
    cols = q.shape[1] * 8
    return np.repeat(_f16(s), GROUP, axis=1) * codes(q, cols) + np.repeat(_f16(b), GROUP, axis=1)


def merged_weights(q, s, b, lora_b, lora_a, alpha_over_r) -> np.ndarray:
    """w' = (s*q + b) + alpha * sum_k B[i,k] A[k,c] in fp64, the rank sum written
    out term by term (each term is exact in fp64)."""
    w = dequant64(q, s, b)
    rows, cols = w.shape
    B = _f16(lora_b).reshape(rows, -1)
    A = _f16(lora_a).reshape(-1, cols)
    t = np.zeros((rows, cols), dtype=np.float64)
    for k in range(A.shape[0]):
        t += B[:, k:k + 1] * A[k:k + 1, :]
    return w + float(alpha_over_r) * t


def group_scale_bias(w: np.ndarray):
    """Per (row, group) of fp64 w: (range / 15 in fp64, s' fp16, b' fp16)."""
    rows, cols = w.shape
    g = w.reshape(rows, cols // GROUP, GROUP)
    exact = (g.max(axis=2) - g.min(axis=2)) / 15.0
    return exact, exact.astype(np.float16), g.min(axis=2).astype(np.float16)


def quotients(w: np.ndarray, s16: np.ndarray, b16: np.ndarray) -> np.ndarray:
    """(w' - b') / s' in fp64 for every weight, given per-group fp16 s', b'
    (float16 arrays [rows][groups]); NaN where s' = 0."""
    rows, cols = w.shape
    sf = np.repeat(np.asarray(s16, dtype=np.float16).astype(np.float64), GROUP, axis=1)
    bf = np.repeat(np.asarray(b16, dtype=np.float16).astype(np.float64), GROUP, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(sf == 0, np.nan, (w - bf) / np.where(sf == 0, 1.0, sf))


def codes_from_quotients(u: np.ndarray) -> np.ndarray:
    """clamp(round_half_even(u), 0, 15), 0 where u is NaN (a constant group)."""
    v = np.clip(np.rint(np.nan_to_num(u, nan=0.0)), 0, 15)
    return v.astype(np.uint32)


def requantize(w: np.ndarray):
    """Min/max affine requantisation of fp64 w' (see the module docstring).
    Returns (q, s, b) in the oracle's format."""
    _, s16, b16 = group_scale_bias(w)
    q = codes_from_quotients(quotients(w, s16, b16))
    return pack(q), s16.view(np.uint16).copy(), b16.view(np.uint16).copy()


def merge_requant(q, s, b, lora_b, lora_a, alpha_over_r):
    """The merged matrix: requantize(merged_weights(...))."""
    return requantize(merged_weights(q, s, b, lora_b, lora_a, alpha_over_r))


def boundary_distance(u: np.ndarray) -> np.ndarray:
    """Distance of each quotient to the nearest half-integer (where rounding
    flips); +inf where u is NaN."""
    return np.where(np.isnan(u), np.inf, np.abs(np.abs(u - np.floor(u)) - 0.5))


def scale_boundary_distance(exact: np.ndarray) -> np.ndarray:
    """Relative distance of range / 15 to the nearest point where its fp16
    rounding flips (the midpoint between two adjacent fp16 values)."""
    h = exact.astype(np.float16)
    lo = np.where(h.astype(np.float64) <= exact, h, np.nextafter(h, np.float16(-np.inf)))
    hi = np.nextafter(lo, np.float16(np.inf))
    mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2.0
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(exact == 0, np.inf, np.abs(exact - mid) / np.abs(exact))


def retention(base, merged, lora_b, lora_a, alpha_over_r) -> float:
    """1 - |U - M| / |U - B| (Frobenius norms, fp64): B the base weights, U = B +
    alpha * lora_b @ lora_a (the unmerged delta, exact), M the merged matrix."""
    Bw = dequant64(*base)
    Bm = _f16(lora_b).reshape(Bw.shape[0], -1)
    Am = _f16(lora_a).reshape(-1, Bw.shape[1])
    U = Bw + float(alpha_over_r) * (Bm @ Am)
    M = dequant64(*merged)
    return float(1.0 - np.linalg.norm(U - M) / np.linalg.norm(U - Bw))
