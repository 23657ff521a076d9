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
rule; this follows the plainest reading of the stacks' affine format:
scale = (max - min) / 15, bias = min, codes rounded half to even and clamped
to 0..15, scale and bias stored as fp16. The merged codes are an integer
decision taken from fp32 values, so it is taken in fp32 here, each operation
rounded to nearest on its own (numpy float32 arithmetic), in the order the
kernel uses: w = s*q + b; t = sum_k B[i,k]*A[k,c] in k order; w' = w + a*t.

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


def merged_weights_f32(q, s, b, lora_b, lora_a, alpha_over_r) -> np.ndarray:
    """w' = (s*q + b) + alpha * sum_k B[i,k] A[k,c], fp32, every step rounded."""
    rows = q.shape[0]
    cols = q.shape[1] * 8
    s32 = np.asarray(s, dtype=np.uint16).view(np.float16).astype(np.float32)
    b32 = np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)
    cq = codes(q, cols).astype(np.float32)
    se = np.repeat(s32, GROUP, axis=1)
    be = np.repeat(b32, GROUP, axis=1)
    w = (se * cq).astype(np.float32)
    w = (w + be).astype(np.float32)
    B = np.asarray(lora_b, dtype=np.uint16).view(np.float16).astype(np.float32).reshape(rows, -1)
    A = np.asarray(lora_a, dtype=np.uint16).view(np.float16).astype(np.float32).reshape(-1, cols)
    t = np.zeros((rows, cols), dtype=np.float32)
    for k in range(A.shape[0]):
        t = (t + (B[:, k:k + 1] * A[k:k + 1, :]).astype(np.float32)).astype(np.float32)
    a = np.float32(alpha_over_r)
    return (w + (a * t).astype(np.float32)).astype(np.float32)


def requantize(w: np.ndarray):
    """Per (row, 64-column group) of fp32 w: s' = fp16((max-min)/15), b' = fp16(min),
    q' = clamp(rint((w - b') / s'), 0, 15) (0 where s' is 0). Returns (q, s, b) in
    the oracle's format."""
    rows, cols = w.shape
    g = w.reshape(rows, cols // GROUP, GROUP)
    hi = g.max(axis=2)
    lo = g.min(axis=2)
    s32 = ((hi - lo).astype(np.float32) / np.float32(15.0)).astype(np.float32)
    s16 = s32.astype(np.float16)
    b16 = lo.astype(np.float16)
    sf = s16.astype(np.float32)[:, :, None]
    bf = b16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.rint(((g - bf).astype(np.float32) / np.where(sf == 0, np.float32(1), sf)).astype(np.float32))
    v = np.clip(v, 0, 15)
    v = np.where(sf == 0, 0, v).astype(np.uint32).reshape(rows, cols)
    return pack(v), s16.view(np.uint16).copy(), b16.view(np.uint16).copy()


def merge_requant(q, s, b, lora_b, lora_a, alpha_over_r):
    """The merged matrix: requantize(merged_weights_f32(...))."""
    return requantize(merged_weights_f32(q, s, b, lora_b, lora_a, alpha_over_r))


def dequant64(q, s, b) -> np.ndarray:
    """s*q + b in fp64 (exact for fp16 s, b and 4-bit q)."""
    cols = q.shape[1] * 8
    s64 = np.asarray(s, dtype=np.uint16).view(np.float16).astype(np.float64)
    b64 = np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.repeat(s64, GROUP, axis=1) * codes(q, cols) + np.repeat(b64, GROUP, axis=1)


def retention(base, merged, lora_b, lora_a, alpha_over_r) -> float:
    """1 - |U - M| / |U - B| (Frobenius norms, fp64): B the base weights, U = B +
    alpha * lora_b @ lora_a (the unmerged delta, exact), M the merged matrix."""
    Bw = dequant64(*base)
    Bm = np.asarray(lora_b, dtype=np.uint16).view(np.float16).astype(np.float64).reshape(Bw.shape[0], -1)
    Am = np.asarray(lora_a, dtype=np.uint16).view(np.float16).astype(np.float64).reshape(-1, Bw.shape[1])
    U = Bw + float(alpha_over_r) * (Bm @ Am)
    M = dequant64(*merged)
    return float(1.0 - np.linalg.norm(U - M) / np.linalg.norm(U - Bw))
