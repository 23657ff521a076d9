"""Seeded synthetic inputs for the routed-expert int4 SwiGLU hot path.

This module is the only code that both the CPU oracle side and the HIP side
use. It draws random numbers and packs bytes; it holds none of the method's
arithmetic (no dequantisation, routing, SwiGLU, head or slot rule).

Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-based: the i-th 64-bit draw of a
stream with key k is ``fin(k + (i + 1) * GAMMA)`` where ``fin`` is SplitMix64's
output mixing function. Stream keys fold identifiers through the same function,
so any tensor of any expert can be regenerated on its own, in any order, on the
CPU (numpy, here) or on the GPU (``e0inputs/csrc/fill.hip``), bit for bit.

Value recipes (every step is exact or a single IEEE round-to-nearest-even):

* uniform24(d)   = (d >> 40) * 2**-24                in [0, 1), exact in fp32
* normal(key, i) = (sum of the twelve 16-bit chunks of draws 3i..3i+2) * 2**-16 - 6
                   (Irwin-Hall: mean 0, variance 1, bounded by 6; exact in fp32).
                   This stands for "N(0,1)" so that both generators agree exactly.
* int4 codes     : each 64-bit draw supplies two little-endian uint32 words of
                   8 nibbles each; nibbles are uniform on 0..15.
* scale          : fp16( fp32(0.005 + fp32(0.015 * u)) )
* bias           : fp16( -8 * fp32(s * fp32(1 + fp32(fp32(0.2 * v) - 0.1))) )
                   i.e. -8 s (1 + U(-0.1, 0.1)) with s the fp16 scale.
"""
from __future__ import annotations

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB
_M64 = (1 << 64) - 1

# Stream tags (first identifier folded into every key).
TAG_EXPERT = 1        # ids: layer, expert, matrix (0 gate, 1 up, 2 down), part (0 q, 1 scale, 2 bias)
TAG_ACT = 2           # ids: step, layer, token
TAG_LOGITS = 3        # ids: step, layer, token
TAG_ROUTER = 4        # ids: layer
TAG_HEAD = 5          # ids: head, tensor
TAG_LORA = 6          # ids: layer, projection, A/B
TAG_SHARED = 7        # ids: layer, matrix, part
TAG_TARGETS = 8       # ids: step, owner layer
TAG_PERM = 9          # ids: (none)
TAG_REDRAW = 10       # ids: ... attempt
TAG_NORM = 11         # ids: layer
TAG_RESID = 12        # ids: step


def _fin_int(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * _C1) & _M64
    z = ((z ^ (z >> 27)) * _C2) & _M64
    return z ^ (z >> 31)


def _fin(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= np.uint64(_C1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(_C2)
    z ^= z >> np.uint64(31)
    return z


def stream_key(seed: int, *ids: int) -> int:
    """Key of the stream named by (seed, ids...): h = fin(seed + G); h = fin((h ^ id) + G)."""
    h = _fin_int(seed + GAMMA)
    for i in ids:
        h = _fin_int(((h ^ (int(i) & _M64)) + GAMMA) & _M64)
    return h


def draws(key: int, n: int, start: int = 0) -> np.ndarray:
    """Draws start..start+n-1 of stream ``key`` as uint64."""
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + i * np.uint64(GAMMA)
    return _fin(z)


def uniform24(d: np.ndarray) -> np.ndarray:
    return (d >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)


def normal(key: int, n: int, start: int = 0) -> np.ndarray:
    """n Irwin-Hall(12) normals as exact fp32 values (see module doc)."""
    d = draws(key, 3 * n, 3 * start).reshape(n, 3)
    tot = np.zeros(n, dtype=np.int64)
    for j in range(3):
        w = d[:, j]
        for c in range(4):
            tot += ((w >> np.uint64(16 * c)) & np.uint64(0xFFFF)).astype(np.int64)
    return (tot.astype(np.float32) * np.float32(2.0 ** -16)) - np.float32(6.0)


def normal_f16(key: int, n: int, std: float = 1.0) -> np.ndarray:
    z = normal(key, n)
    if std != 1.0:
        z = np.float32(std) * z
    return z.astype(np.float16)


# ---------------------------------------------------------------------------
# int4 group-64 expert matrices
# ---------------------------------------------------------------------------

GROUP = 64


def quant_matrix(key_q: int, key_s: int, key_b: int, rows: int, cols: int):
    """Codes, scales and biases of one [rows][cols] matrix.

    Returns (q uint32 [rows, cols/8], s fp16-bits uint16 [rows, cols/64],
    b fp16-bits uint16 [rows, cols/64]).
    """
    assert cols % GROUP == 0
    nw = rows * cols // 8
    q = draws(key_q, (nw + 1) // 2).view(np.uint32)[:nw].reshape(rows, cols // 8)
    ng = rows * cols // GROUP
    u = uniform24(draws(key_s, ng))
    s32 = np.float32(0.005) + np.float32(0.015) * u
    s16 = s32.astype(np.float16)
    v = uniform24(draws(key_b, ng))
    t = np.float32(1.0) + (np.float32(0.2) * v - np.float32(0.1))
    b32 = np.float32(-8.0) * (s16.astype(np.float32) * t)
    b16 = b32.astype(np.float16)
    return (np.ascontiguousarray(q),
            s16.view(np.uint16).reshape(rows, cols // GROUP).copy(),
            b16.view(np.uint16).reshape(rows, cols // GROUP).copy())


def expert_matrix(seed: int, layer: int, expert: int, mat: int, d: int, f: int, tag: int = TAG_EXPERT):
    """Matrix ``mat`` (0 gate [f][d], 1 up [f][d], 2 down [d][f]) of one expert."""
    rows, cols = (f, d) if mat < 2 else (d, f)
    return quant_matrix(stream_key(seed, tag, layer, expert, mat, 0),
                        stream_key(seed, tag, layer, expert, mat, 1),
                        stream_key(seed, tag, layer, expert, mat, 2), rows, cols)


def expert(seed: int, layer: int, expert_id: int, d: int, f: int, tag: int = TAG_EXPERT):
    """The three matrices of one expert: [(q, s, b) gate, up, down]."""
    return [expert_matrix(seed, layer, expert_id, m, d, f, tag) for m in range(3)]


# ---------------------------------------------------------------------------
# Bundle layout: one expert = 9 contiguous parts
#   [gate q | gate s | gate b | up q | up s | up b | down q | down s | down b]
# q parts are uint32 words [rows][cols/8] (8 codes each, code c at bits
# 4*(c%8) of word c/8); s and b parts are fp16 bit patterns stored in tiles of
# 8 rows, [rows/8][cols/64][8]: the scale of row r, group g (columns 64g ..
# 64g+63) is element ((r/8)*(cols/64) + g)*8 + r%8, so the 8 rows of a tile in
# one group are 16 contiguous bytes and a tile's groups follow each other.
# The arrays returned by quant_matrix are [rows][cols/64].
# ---------------------------------------------------------------------------

def part_sizes(d: int, f: int):
    qb = d * f // 2
    sb = d * f // GROUP * 2
    return [qb, sb, sb] * 3


def part_offsets(d: int, f: int):
    offs, o = [], 0
    for sz in part_sizes(d, f):
        offs.append(o)
        o += sz
    return offs


def bundle_bytes(d: int, f: int) -> int:
    return sum(part_sizes(d, f))


def _tile8(a: np.ndarray) -> np.ndarray:
    """[rows][ngrp] -> [rows/8][ngrp][8] (the bundle order of scales and biases)."""
    rows, ngrp = a.shape
    return a.reshape(rows // 8, 8, ngrp).transpose(0, 2, 1)


def _untile8(flat: np.ndarray, rows: int, ngrp: int) -> np.ndarray:
    return np.ascontiguousarray(flat.reshape(rows // 8, ngrp, 8).transpose(0, 2, 1).reshape(rows, ngrp))


def pack_bundle(mats, d: int, f: int) -> np.ndarray:
    """uint8 bundle of one expert from [(q, s, b)] * 3."""
    out = np.empty(bundle_bytes(d, f), dtype=np.uint8)
    offs = part_offsets(d, f)
    j = 0
    for (q, s, b) in mats:
        for arr in (q, _tile8(s), _tile8(b)):
            raw = np.ascontiguousarray(arr).view(np.uint8).ravel()
            out[offs[j]:offs[j] + raw.size] = raw
            j += 1
    return out


def unpack_bundle(buf: np.ndarray, d: int, f: int):
    """Inverse of pack_bundle."""
    offs = part_offsets(d, f)
    sizes = part_sizes(d, f)
    mats = []
    for m in range(3):
        rows, cols = (f, d) if m < 2 else (d, f)
        q = buf[offs[3 * m]:offs[3 * m] + sizes[3 * m]].view(np.uint32).reshape(rows, cols // 8)
        s = buf[offs[3 * m + 1]:offs[3 * m + 1] + sizes[3 * m + 1]].view(np.uint16)
        b = buf[offs[3 * m + 2]:offs[3 * m + 2] + sizes[3 * m + 2]].view(np.uint16)
        mats.append((q, _untile8(s, rows, cols // GROUP), _untile8(b, rows, cols // GROUP)))
    return mats


def layer_store(seed: int, layer: int, n_experts: int, d: int, f: int, tag: int = TAG_EXPERT) -> np.ndarray:
    """All experts of one layer as contiguous bundles, uint8 [E, bundle]."""
    bb = bundle_bytes(d, f)
    out = np.empty((n_experts, bb), dtype=np.uint8)
    for e in range(n_experts):
        out[e] = pack_bundle(expert(seed, layer, e, d, f, tag), d, f)
    return out
