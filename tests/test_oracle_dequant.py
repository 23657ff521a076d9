"""Oracle pins: fp16 decoding and the int4 affine group-64 decode."""
import json
import os

import numpy as np

import oracle
from e0inputs import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_half_decoding_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.half(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_dequant_golden_words():
    g = json.load(open(os.path.join(GOLD, "dequant_words.json")))
    q = np.zeros((1, 8), dtype=np.uint32)
    q[0, 0] = int(g["word_hex"][0], 16)
    q[0, 1] = int(g["word_hex"][1], 16)
    s = np.array([[int(g["scale_fp16_hex"], 16)]], dtype=np.uint16)
    b = np.array([[int(g["bias_fp16_hex"], 16)]], dtype=np.uint16)
    w = oracle.dequant(q, s, b, 1, 64)
    assert w[0, :16].tolist() == g["expected_first_16"]


def test_dequant_all_codes_and_groups():
    # Every code in every nibble position, with distinct (s, b) per group; the
    # expected value is built by hand from scale*q + bias, groups of 64.
    rows, cols = 3, 192
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=(rows, cols))
    codes[0, :16] = np.arange(16)
    q = np.zeros((rows, cols // 8), dtype=np.uint32)
    for c in range(cols):
        q[:, c // 8] |= (codes[:, c].astype(np.uint32) << np.uint32(4 * (c % 8)))
    s = rng.uniform(0.005, 0.02, size=(rows, cols // 64)).astype(np.float16)
    b = (-8 * s.astype(np.float32) * rng.uniform(0.9, 1.1, size=s.shape).astype(np.float32)).astype(np.float16)
    got = oracle.dequant(q, s.view(np.uint16), b.view(np.uint16), rows, cols)
    for r in range(rows):
        for c in range(cols):
            exp = float(s[r, c // 64]) * codes[r, c] + float(b[r, c // 64])
            assert got[r, c] == exp


def test_dequant_is_exact_in_fp32():
    # With fp16 scale and bias and codes 0..15, s*q + b needs at most 24
    # significant bits, so an fp32 dequantisation loses nothing.
    q, s, b = gen.expert_matrix(1002, 0, 0, 0, 2048, 512)
    w = oracle.dequant(q, s, b, 512, 2048)
    codes = np.stack([(q >> (4 * i)) & 15 for i in range(8)], -1).reshape(512, 2048).astype(np.float32)
    sf = np.repeat(s.view(np.float16).astype(np.float32), 64, axis=1)
    bf = np.repeat(b.view(np.float16).astype(np.float32), 64, axis=1)
    w32 = sf * codes + bf
    assert np.array_equal(w32.astype(np.float64), w)
