"""Oracle pins: softmax-top-K (renormalised) and sigmoid-group routing.

Pinned against textbook reductions, brute force and the invariants the pages
state (softmax-top-K weights sum to 1; sigmoid-group weights sum to s)."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from e0inputs import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _logits(T, E, seed):
    return np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)


@pytest.mark.parametrize("E,K", [(16, 4), (256, 4), (8, 1), (64, 8)])
def test_softmax_topk_indices_are_argsort(E, K):
    lg = _logits(32, E, E + K)
    idx, w = oracle.softmax_topk(lg, K)
    ref = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :K]
    assert np.array_equal(idx, ref)
    assert np.allclose(w.sum(1), 1.0, atol=1e-12, rtol=0)


def test_softmax_topk_k1_and_k_equals_e():
    lg = _logits(16, 16, 1)
    idx, w = oracle.softmax_topk(lg, 1)
    assert np.all(w == 1.0)
    idx, w = oracle.softmax_topk(lg, 16)
    full = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(np.take_along_axis(full, idx, 1), w, rtol=1e-13, atol=0)


def test_softmax_topk_weights_are_renormalised_probabilities():
    lg = _logits(8, 32, 2)
    idx, w = oracle.softmax_topk(lg, 4)
    for t in range(8):
        g = softmax(lg[t].astype(np.float64))
        sel = g[idx[t]]
        assert np.allclose(w[t], sel / sel.sum(), rtol=1e-13, atol=0)


def test_ties_go_to_the_lower_id():
    lg = np.zeros((1, 16), dtype=np.float32)
    lg[0, [9, 3, 12, 5]] = 2.0
    idx, _ = oracle.softmax_topk(lg, 3)
    assert idx[0].tolist() == [3, 5, 9]
    idx, _ = oracle.softmax_topk(np.zeros((1, 16), np.float32), 4)
    assert idx[0].tolist() == [0, 1, 2, 3]


def _brute_sigmoid_group(l, K, n, G, s, eps):
    """Kept groups = the G-subset with the largest total group score, group
    score = the largest sum of any two distinct members' sigmoid."""
    E = l.size
    per = E // n
    sig = expit(l.astype(np.float64))
    score = []
    for g in range(n):
        mem = sig[g * per:(g + 1) * per]
        score.append(max(a + b for a, b in itertools.combinations(mem, 2)) if per > 1 else mem[0])
    best = max(itertools.combinations(range(n), G), key=lambda c: sum(score[i] for i in c))
    kept = [e for g in best for e in range(g * per, (g + 1) * per)]
    order = sorted(kept, key=lambda e: (-sig[e], e))[:K]
    ws = np.array([sig[e] for e in order])
    return order, s * ws / (ws.sum() + eps)


@pytest.mark.parametrize("E,K,n,G", [(16, 4, 4, 2), (32, 8, 8, 4), (24, 3, 6, 3)])
def test_sigmoid_group_brute_force(E, K, n, G):
    lg = _logits(24, E, 10 * E + K)
    idx, w = oracle.sigmoid_group(lg, K, n, G, 2.5)
    for t in range(lg.shape[0]):
        order, ww = _brute_sigmoid_group(lg[t], K, n, G, 2.5, 1e-20)
        assert idx[t].tolist() == order
        assert np.allclose(w[t], ww, rtol=1e-13, atol=0)


def test_sigmoid_group_all_groups_is_plain_sigmoid_topk():
    lg = _logits(16, 128, 5)
    idx, w = oracle.sigmoid_group(lg, 8, 8, 8, 1.0)
    sig = expit(lg.astype(np.float64))
    ref = np.argsort(-sig, axis=1, kind="stable")[:, :8]
    assert np.array_equal(idx, ref)


def test_sigmoid_group_weights_sum_to_scale():
    g = json.load(open(os.path.join(GOLD, "pages_constants.json")))["tier8"]
    lg = _logits(64, g["experts"], 9)
    idx, w = oracle.sigmoid_group(lg, g["top_k"], g["n_groups"], g["topk_groups"], g["scale"])
    assert np.allclose(w.sum(1), g["scale"], rtol=1e-14, atol=0)
    # only kept groups contribute
    per = g["experts"] // g["n_groups"]
    assert all(len(set((idx[t] // per).tolist())) <= g["topk_groups"] for t in range(64))


def test_sigmoid_group_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.sigmoid_group(_logits(1, 30, 0), 4, 8, 4, 2.5)
    with pytest.raises(ValueError):
        oracle.sigmoid_group(_logits(1, 16, 0), 9, 8, 4, 2.5)


def test_margins():
    lg = _logits(20, 64, 3)
    cfg = W.scaled(W.DECODE35, E=64)
    m = oracle.route_margin(lg, cfg)
    v = -np.sort(-lg.astype(np.float64), axis=1)[:, :5]
    assert m == np.min(v[:, :-1] - v[:, 1:])
    lg2 = lg.copy()
    lg2[0, np.argmax(lg2[0])] = np.sort(lg2[0])[-2]
    assert oracle.route_margin(lg2, cfg) == 0.0
    cfg8 = W.scaled(W.DECODE8_B1, E=64)
    assert oracle.route_margin(lg, cfg8) > 0
