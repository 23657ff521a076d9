"""Oracle pins: the expert SwiGLU, the weighted combine, the three orderings,
the slot rule, the prerouter head and the unmerged LoRA."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import erf

import oracle
from e0inputs import gen, workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")
CFG = W.TINY


def _dense(mats, d, f):
    """Independent numpy decode of the three matrices (fp64)."""
    out = []
    for m, (q, s, b) in enumerate(mats):
        rows, cols = (f, d) if m < 2 else (d, f)
        codes = np.stack([(q >> np.uint32(4 * i)) & np.uint32(15) for i in range(8)], -1).reshape(rows, cols)
        sf = np.repeat(s.view(np.float16).astype(np.float64), 64, axis=1)
        bf = np.repeat(b.view(np.float16).astype(np.float64), 64, axis=1)
        out.append(sf * codes + bf)
    return out


def _swiglu(G, U, D, x):
    g, u = G @ x, U @ x
    return D @ (g / (1 + np.exp(-g)) * u)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _tiny_layer(cfg=CFG):
    experts = [gen.expert(cfg.seed, 0, e, cfg.d, cfg.f) for e in range(cfg.E)]
    x = W.activations(cfg, 0, 0)
    lg = oracle.router_logits(x, W.router_weights(cfg, 0))
    idx, w = oracle.route(lg, cfg)
    return experts, x, idx, w


def test_expert_ffn_is_dense_swiglu():
    d, f = CFG.d, CFG.f
    mats = gen.expert(CFG.seed, 0, 5, d, f)
    x = W.activations(CFG, 0, 0)[0]
    G, U, D = _dense(mats, d, f)
    ref = _swiglu(G, U, D, x.astype(np.float64))
    got = oracle.expert_ffn(mats, x, d, f)
    assert _rel(got, ref) < 1e-13


def test_router_logits_is_a_gemv():
    x = W.activations(CFG, 0, 0)
    wr = W.router_weights(CFG, 0)
    got = oracle.router_logits(x, wr)
    ref = (x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32)
    assert np.array_equal(got, ref)


def test_single_expert_weight_one_equals_dense():
    experts, x, _, _ = _tiny_layer()
    ex = oracle.Experts(experts)
    idx = np.array([[7]], dtype=np.int32)
    y, err = oracle.moe_exact(ex, CFG.d, CFG.f, x[:1], idx, np.ones((1, 1)))
    G, U, D = _dense(experts[7], CFG.d, CFG.f)
    assert err == 0 and _rel(y[0], _swiglu(G, U, D, x[0].astype(np.float64))) < 1e-13


def test_weighted_combine_matches_dense_sum():
    experts, x, idx, w = _tiny_layer()
    y, err = oracle.moe_exact(oracle.Experts(experts), CFG.d, CFG.f, x, idx, w)
    assert err == 0
    dense = [_dense(m, CFG.d, CFG.f) for m in experts]
    for t in range(CFG.B):
        ref = sum(w[t, k] * _swiglu(*dense[idx[t, k]], x[t].astype(np.float64)) for k in range(CFG.K))
        assert _rel(y[t], ref) < 1e-13


def test_three_orderings_are_bitwise_equal():
    experts, x, idx, w = _tiny_layer()
    ex = oracle.Experts(experts)
    y_exact, e1 = oracle.moe_exact(ex, CFG.d, CFG.f, x, idx, w)
    y_sorted, e2, perm = oracle.moe_sorted(ex, CFG.d, CFG.f, x, idx, w)
    # staged: a pool of S slots filled by the slot rule from an empty pool
    slot_of = np.full(CFG.E, -1, np.int32)
    expert_of = np.full(CFG.E, -1, np.int32)  # S = E here so any routing fits
    rc, copies = oracle.slot_update(CFG.E, CFG.E, np.unique(idx), [], slot_of, expert_of)
    assert rc == 0
    pool = [experts[e] if e >= 0 else experts[0] for e in expert_of]
    y_staged, e3 = oracle.moe_staged(oracle.Experts(pool), slot_of, CFG.E, CFG.d, CFG.f, x, idx, w)
    assert e1 == e2 == e3 == 0
    assert np.array_equal(y_exact.view(np.uint64), y_sorted.view(np.uint64))
    assert np.array_equal(y_exact.view(np.uint64), y_staged.view(np.uint64))
    # the sorted order is by (expert, token), stable
    keys = [(idx.ravel()[p], p) for p in perm]
    assert keys == sorted(keys)


def test_negative_control_gate_up_swap_and_row_shift():
    experts, x, idx, w = _tiny_layer()
    y, _ = oracle.moe_exact(oracle.Experts(experts), CFG.d, CFG.f, x, idx, w)
    swapped = [[m[1], m[0], m[2]] for m in experts]
    y2, _ = oracle.moe_exact(oracle.Experts(swapped), CFG.d, CFG.f, x, idx, w)
    assert _rel(y2, y) > 0.5
    shifted = [[m[0], m[1], tuple(np.roll(a, 1, axis=0) for a in m[2])] for m in experts]
    y3, _ = oracle.moe_exact(oracle.Experts(shifted), CFG.d, CFG.f, x, idx, w)
    assert _rel(y3, y) > 0.5


def test_staged_flags_missing_and_bad_ids():
    experts, x, idx, w = _tiny_layer()
    slot_of = np.full(CFG.E, -1, np.int32)
    y, err = oracle.moe_staged(oracle.Experts(experts[:4]), slot_of, CFG.E, CFG.d, CFG.f, x, idx, w)
    assert err == 2 and np.all(y == 0)
    bad = idx.copy()
    bad[0, 0] = CFG.E
    y, err = oracle.moe_exact(oracle.Experts(experts), CFG.d, CFG.f, x, bad, w)
    assert err & 1


def test_slot_rule_walkthrough():
    g = json.load(open(os.path.join(GOLD, "slot_rule_walkthrough.json")))
    E, S = g["E"], g["S"]
    slot_of = np.full(E, -1, np.int32)
    expert_of = np.full(S, -1, np.int32)
    for st in g["steps"]:
        rc, copies = oracle.slot_update(E, S, st["want"], st["keep"], slot_of, expert_of)
        if "error" in st:
            assert rc == st["error"]
            continue
        assert rc == 0
        assert [list(c) for c in copies] == st["copies"]
        assert expert_of.tolist() == st["expert_of"]
        for s, e in enumerate(expert_of):
            if e >= 0:
                assert slot_of[e] == s
        assert np.sum(slot_of >= 0) == np.sum(expert_of >= 0)


def test_slot_rule_invariants_random():
    rng = np.random.default_rng(4)
    E, S, K = 32, 8, 4
    slot_of = np.full(E, -1, np.int32)
    expert_of = np.full(S, -1, np.int32)
    cur = np.array([], dtype=np.int32)
    for _ in range(300):
        nxt = rng.choice(E, K, replace=False).astype(np.int32)
        before = expert_of.copy()
        resident = set(int(e) for e in before if e >= 0)
        rc, copies = oracle.slot_update(E, S, nxt, cur, slot_of, expert_of)
        assert rc == 0
        assert len(copies) == len(set(nxt.tolist()) - resident)
        assert all(slot_of[e] >= 0 and expert_of[slot_of[e]] == e for e in nxt)
        for s in range(S):  # slots holding in-use experts were not touched
            if before[s] in set(cur.tolist()):
                assert expert_of[s] == before[s]
        for s, e in copies:  # lowest free slot was taken
            assert e not in resident
        cur = nxt


def test_head_feature_layout_toy_example():
    g = json.load(open(os.path.join(GOLD, "pages_constants.json")))["toy_head"]
    h = np.arange(1, g["d_model"] + 1).astype(np.float16) / 8
    feat = oracle.head_feature(h, g["E"], np.array([1]), np.array([0]), g["K"])
    assert feat.size == g["input_dim"]
    assert feat[:8].tolist() == h.astype(np.float64).tolist()
    assert feat[8:12].tolist() == g["one_hot_now"]
    assert feat[12:16].tolist() == g["one_hot_prev"]
    f0 = oracle.head_feature(h, g["E"], np.array([1]), None, g["K"])
    assert f0[12:].tolist() == [0, 0, 0, 0]


def test_head_dimension_35b():
    g = json.load(open(os.path.join(GOLD, "pages_constants.json")))["head"]
    cfg = W.PREROUTED35
    hd = W.head(cfg, 3)
    assert hd.fc1_w.shape == (g["hidden"], g["input_dim"])


def _zero_head(E, d, hid, lin):
    return W.Head(fc1_w=np.zeros((hid, d + 2 * E), np.float16), fc1_b=np.zeros(hid, np.float16),
                  fc2_w=np.zeros((E, hid), np.float16), fc2_b=np.zeros(E, np.float16), lin_w=lin)


def test_head_with_zero_mlp_is_the_next_router():
    # fc1 = fc2 = 0: the head reduces to its warm start, the next layer's
    # router applied to this hidden state.
    cfg = W.scaled(W.PREROUTED35, d=256, E=32)
    lin = W.router_weights(cfg, 2)
    hd = _zero_head(cfg.E, cfg.d, 64, lin)
    h = W.activations(cfg, 0, 0)[0]
    o = oracle.head_logits(hd, h, np.array([1, 2, 3, 4]), np.array([5, 6, 7, 8]), 4)
    # gelu(0) = 0, so o = lin h exactly up to summation order
    assert np.allclose(o, lin.astype(np.float64) @ h.astype(np.float64), rtol=0, atol=1e-12)


@pytest.mark.parametrize("a", [-3.0, -0.5, 0.0, 0.25, 1.0, 2.5])
def test_head_gelu_is_erf_gelu(a):
    E, d, hid = 8, 64, 16
    hd = _zero_head(E, d, hid, np.zeros((E, d), np.float16))
    hd.fc1_b[0] = np.float16(a)
    hd.fc2_w[0, 0] = np.float16(1.0)
    o = oracle.head_logits(hd, np.zeros(d, np.float16), np.array([0]), None, 1)
    av = float(np.float16(a))
    assert o[0] == pytest.approx(0.5 * av * (1 + math.erf(av / math.sqrt(2))), rel=1e-15, abs=1e-300)
    assert np.all(o[1:] == 0)


def test_head_khot_columns_enter_fc1():
    E, d, hid = 8, 16, 4
    hd = _zero_head(E, d, hid, np.zeros((E, d), np.float16))
    hd.fc1_w[0, d + 3] = np.float16(1.0)       # current-token one-hot of expert 3
    hd.fc1_w[1, d + E + 5] = np.float16(1.0)   # previous-token one-hot of expert 5
    hd.fc2_w[0, 0] = np.float16(1.0)
    hd.fc2_w[1, 1] = np.float16(1.0)
    gelu1 = 0.5 * (1 + math.erf(1 / math.sqrt(2)))
    o = oracle.head_logits(hd, np.zeros(d, np.float16), np.array([3, 4]), np.array([5, 6]), 2)
    assert o[0] == pytest.approx(gelu1) and o[1] == pytest.approx(gelu1)
    o = oracle.head_logits(hd, np.zeros(d, np.float16), np.array([4, 2]), np.array([6, 1]), 2)
    assert o[0] == 0 and o[1] == 0


def test_head_random_matches_numpy():
    cfg = W.scaled(W.PREROUTED35, d=128, E=32)
    hid = 64
    rng = np.random.default_rng(1)
    hd = W.Head(fc1_w=(rng.standard_normal((hid, cfg.d + 2 * cfg.E)) * 0.05).astype(np.float16),
                fc1_b=(rng.standard_normal(hid) * 0.05).astype(np.float16),
                fc2_w=(rng.standard_normal((cfg.E, hid)) * 0.05).astype(np.float16),
                fc2_b=(rng.standard_normal(cfg.E) * 0.05).astype(np.float16),
                lin_w=(rng.standard_normal((cfg.E, cfg.d)) * 0.05).astype(np.float16))
    h = rng.standard_normal(cfg.d).astype(np.float16)
    cur, prev = np.array([3, 9, 1, 30]), np.array([9, 2, 7, 11])
    feat = np.concatenate([h.astype(np.float64), np.zeros(2 * cfg.E)])
    feat[cfg.d + cur] = 1
    feat[cfg.d + cfg.E + prev] = 1
    a = hd.fc1_w.astype(np.float64) @ feat + hd.fc1_b.astype(np.float64)
    gl = 0.5 * a * (1 + erf(a / np.sqrt(2)))
    ref = hd.fc2_w.astype(np.float64) @ gl + hd.fc2_b.astype(np.float64) + hd.lin_w.astype(np.float64) @ h.astype(np.float64)
    o = oracle.head_logits(hd, h, cur, prev, 4)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_lora_zero_b_is_base():
    cfg = W.scaled(W.PREROUTED35, d=256, shared_f=128)
    mats = W.shared_expert(cfg, 0)
    lo = W.lora(cfg, 0)
    zero = [(a, np.zeros_like(b)) for a, b in lo]
    x = W.activations(cfg, 0, 0)[0]
    y0 = oracle.shared_lora(mats, None, cfg.lora_r, 2.0, x, cfg.d, cfg.shared_f)
    y1 = oracle.shared_lora(mats, zero, cfg.lora_r, 2.0, x, cfg.d, cfg.shared_f)
    assert np.array_equal(y0, y1)


def test_lora_unmerged_equals_merged_in_fp64():
    cfg = W.scaled(W.PREROUTED35, d=256, shared_f=128)
    mats = W.shared_expert(cfg, 1)
    lo = W.lora(cfg, 1)
    x = W.activations(cfg, 0, 1)[0]
    y = oracle.shared_lora(mats, lo, cfg.lora_r, 2.0, x, cfg.d, cfg.shared_f)
    G, U, D = _dense(mats, cfg.d, cfg.shared_f)
    merged = [Wm + 2.0 * (b.astype(np.float64) @ a.astype(np.float64)) for Wm, (a, b) in zip((G, U, D), lo)]
    ref = _swiglu(*merged, x.astype(np.float64))
    assert _rel(y, ref) < 1e-12
    base = oracle.shared_lora(mats, None, cfg.lora_r, 2.0, x, cfg.d, cfg.shared_f)
    assert _rel(y, base) > 1e-3  # the delta is not negligible


def test_decode_layers_threads_agree():
    cfg = W.scaled(W.TINY, L=3)
    L, S = cfg.L, 8
    pools, slot_of, xs, idxs, ws = [], [], [], [], []
    for l in range(L):
        experts = [gen.expert(cfg.seed, l, e, cfg.d, cfg.f) for e in range(cfg.E)]
        x = W.activations(cfg, 0, l)[:2]
        idx, w = oracle.softmax_topk(W.given_logits(cfg, 0, l)[:2].astype(np.float32), cfg.K)
        so = np.full(cfg.E, -1, np.int32)
        eo = np.full(S, -1, np.int32)
        rc, _ = oracle.slot_update(cfg.E, S, np.unique(idx), [], so, eo)
        assert rc == 0
        pools += [experts[e] if e >= 0 else experts[0] for e in eo]
        slot_of.append(so)
        xs.append(x)
        idxs.append(idx)
        ws.append(w)
    P = oracle.Experts(pools)
    a = oracle.decode_layers(P, S, np.stack(slot_of), cfg.E, cfg.d, cfg.f, np.stack(xs), np.stack(idxs), np.stack(ws), 1)
    b = oracle.decode_layers(P, S, np.stack(slot_of), cfg.E, cfg.d, cfg.f, np.stack(xs), np.stack(idxs), np.stack(ws), 3)
    assert a[1] == 0 and np.array_equal(a[0], b[0])


def test_moe_by_expert_equals_per_pair_loop():
    # The per-expert matrix-product form (used for full-size GPU parity) against
    # the C oracle's per-(token, k) loop: same definition, different summation
    # order, so equal to fp64 rounding. An out-of-range id contributes nothing
    # in both.
    cfg = W.scaled(W.TINY, B=37)
    x = W.activations(cfg, 5, 0)
    idx, w = oracle.softmax_topk(W.given_logits(cfg, 5, 0).astype(np.float32), cfg.K)
    idx[3, 1] = cfg.E
    w[3, 1] = 0.0
    mats = [gen.expert(cfg.seed, 0, e, cfg.d, cfg.f) for e in range(cfg.E)]
    ref, err = oracle.moe_exact(oracle.Experts(mats), cfg.d, cfg.f, x, idx, w)
    got = oracle.moe_by_expert(lambda e: mats[e], cfg.E, cfg.d, cfg.f, x, idx, w)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    # a swapped gate/up in the per-expert form is caught
    swapped = oracle.moe_by_expert(lambda e: [mats[e][1], mats[e][0], mats[e][2]], cfg.E, cfg.d, cfg.f, x, idx, w)
    assert np.linalg.norm(swapped - ref) / np.linalg.norm(ref) > 0.1
