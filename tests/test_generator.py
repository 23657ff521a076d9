"""Input generator: determinism, value ranges, and the byte counts the pages print."""
import json
import os

import numpy as np

from e0inputs import gen, workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first outputs of the public reference
    # implementation (Vigna's splitmix64.c, seed 0).
    out = gen.draws(0, 3)
    assert [int(v) for v in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_stream_keys_are_distinct_and_deterministic():
    keys = {gen.stream_key(1002, gen.TAG_EXPERT, l, e, m, p) for l in range(3) for e in range(4)
            for m in range(3) for p in range(3)}
    assert len(keys) == 3 * 4 * 3 * 3
    assert gen.stream_key(5, 1, 2) == gen.stream_key(5, 1, 2)
    a = gen.expert(1002, 3, 7, 256, 128)
    b = gen.expert(1002, 3, 7, 256, 128)
    for (qa, sa, ba), (qb, sb, bb) in zip(a, b):
        assert np.array_equal(qa, qb) and np.array_equal(sa, sb) and np.array_equal(ba, bb)


def test_value_distributions():
    q, s, b = gen.expert_matrix(1001, 0, 0, 0, 2048, 512)
    codes = np.stack([(q >> (4 * i)) & 15 for i in range(8)], -1).ravel()
    counts = np.bincount(codes, minlength=16)
    assert counts.min() > 0.95 * codes.size / 16 and counts.max() < 1.05 * codes.size / 16
    sf = s.view(np.float16).astype(np.float64)
    bf = b.view(np.float16).astype(np.float64)
    assert sf.min() >= 0.005 - 1e-5 and sf.max() <= 0.02 + 1e-5
    r = bf / sf
    assert r.min() >= -8.8 * (1 + 1e-3) and r.max() <= -7.2 * (1 - 1e-3)
    z = gen.normal(77, 200000)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.02 and np.abs(z).max() <= 6


def test_normal_is_exact_fp32():
    z = gen.normal(3, 1000)
    assert np.all(z * 65536 == np.round(z * 65536))


def test_bundle_bytes_match_the_pages():
    g = json.load(open(os.path.join(GOLD, "pages_constants.json")))
    mb = g["moe_bytes"]
    t35 = g["tier35"]
    per_expert = gen.bundle_bytes(2048, 512)
    assert per_expert == W.expert_bytes(2048, 512) == 1_769_472
    assert round(per_expert / 1e6, 2) == mb["per_expert_MB"]
    per_layer = per_expert * t35["experts"]
    assert per_layer == 452_984_832 and round(per_layer / 1e6) == mb["per_layer_MB"]
    total = per_layer * t35["layers"]
    assert round(total / 1e9) == mb["total_GB"]
    assert round(total / 2 ** 30, 1) == mb["total_GiB"]
    assert gen.bundle_bytes(256, 128) == 55_296


def test_pack_unpack_roundtrip():
    mats = gen.expert(1001, 0, 3, 256, 128)
    buf = gen.pack_bundle(mats, 256, 128)
    back = gen.unpack_bundle(buf, 256, 128)
    for (q, s, b), (q2, s2, b2) in zip(mats, back):
        assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(b, b2)
    offs = gen.part_offsets(2048, 512)
    assert all(o % 256 == 0 for o in offs)


def test_head_weight_bytes():
    g = json.load(open(os.path.join(GOLD, "pages_constants.json")))["head"]
    cfg = W.PREROUTED35
    assert cfg.d + 2 * cfg.E == g["input_dim"]
    assert W.HEAD_HIDDEN == g["hidden"]
    assert W.head_weight_bytes(cfg) == 3_416_064


def test_repeat_process():
    cfg = W.PREROUTED35
    s = W.initial_set(cfg, 0)
    assert len(set(s.tolist())) == cfg.K
    kept = tot = 0
    for t in range(1, 400):
        n = W.next_set(cfg, s, t, 0)
        assert len(set(n.tolist())) == cfg.K and n.min() >= 0 and n.max() < cfg.E
        kept += int(np.sum(n == s))
        tot += cfg.K
        s = n
    assert abs(kept / tot - cfg.repeat_p) < 0.05


def test_zipf_bias_is_a_permuted_log_rank():
    cfg = W.PREFILL35
    b = W.popularity_bias(cfg).astype(np.float64)
    ranks = np.exp(-b / cfg.zipf)
    assert np.allclose(np.sort(ranks), np.arange(1, cfg.E + 1), rtol=1e-5)
