"""GPU parity: the generator's GPU fill, and e0_route against the oracle.

Routing indices must match bit for bit; weights within 1e-6 (fp32 softmax /
sigmoid of the same or near-equal logits). Where the logits are computed
(router GEMV) the inputs are redrawn until every decision has a margin of at
least 1e-3 in the oracle's scores, far above fp32 rounding (~1e-6)."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
DELTA = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from int4_gather_swiglu_amd import _lib as E
    E.lib()
    return E


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def test_gpu_fill_matches_numpy_generator():
    T = U.torch()
    for cfg, layer, ids in ((W.TINY, 0, list(range(16))), (W.DECODE35, 3, [0, 77, 255])):
        bb = gen.bundle_bytes(cfg.d, cfg.f)
        buf = U.zeros((len(ids), bb), "uint8")
        from e0inputs import gpu as G
        G.fill_experts(buf.data_ptr(), bb, cfg.seed, layer, ids, cfg.d, cfg.f)
        got = buf.cpu().numpy()
        for i, e in enumerate(ids):
            ref = gen.pack_bundle(gen.expert(cfg.seed, layer, e, cfg.d, cfg.f), cfg.d, cfg.f)
            assert np.array_equal(got[i], ref), (cfg.name, e)
    del T


def _route_given(lg_np, params, fp16=True):
    L, Tn, Ex = lg_np.shape
    K = params.k
    lg = U.f16(lg_np) if fp16 else U.f32(lg_np)
    idx = U.empty((L, Tn, K), "int32")
    w = U.empty((L, Tn, K))
    E().e0_route(params, L, Tn, Ex, lg, fp16, None, None, 0, idx, w, None)
    U.torch().cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


def test_softmax_topk_given_fp16_logits_35b_shapes():
    cfg = W.DECODE35
    steps = 32
    lg = np.stack([np.stack([W.given_logits(cfg, s, l) for l in range(cfg.L)]) for s in range(steps)])
    lg = lg.reshape(steps * cfg.L, 1, cfg.E)
    idx, w = _route_given(lg, E().route_params(0, cfg.K))
    ridx, rw = oracle.softmax_topk(lg.reshape(-1, cfg.E).astype(np.float32), cfg.K)
    assert np.array_equal(idx.reshape(-1, cfg.K), ridx)
    assert np.abs(w.reshape(-1, cfg.K) - rw).max() < 1e-6


def test_ties_resolve_to_lower_id_like_the_oracle():
    lg = np.zeros((1, 4, 64), dtype=np.float16)
    lg[0, 0, [40, 7, 22, 9, 3]] = 1.5
    lg[0, 1, :] = 0.25
    lg[0, 2, [63, 0]] = 2.0
    lg[0, 3, ::2] = -1.0
    idx, w = _route_given(lg, E().route_params(0, 4))
    ridx, rw = oracle.softmax_topk(lg[0].astype(np.float32), 4)
    assert np.array_equal(idx[0], ridx)
    assert idx[0, 0].tolist() == [3, 7, 9, 22]
    assert np.abs(w[0] - rw).max() < 1e-6


@pytest.mark.parametrize("Ex,K", [(16, 1), (16, 16), (100, 7), (1024, 8), (256, 32)])
def test_softmax_topk_edge_shapes(Ex, K):
    rng = np.random.default_rng(Ex * 100 + K)
    lg = rng.standard_normal((2, 33, Ex)).astype(np.float32)
    idx, w = _route_given(lg, E().route_params(0, K), fp16=False)
    ridx, rw = oracle.softmax_topk(lg.reshape(-1, Ex), K)
    assert np.array_equal(idx.reshape(-1, K), ridx)
    assert np.abs(w.reshape(-1, K) - rw).max() < 1e-6


def _tie_free_x(cfg, step, layer, wr):
    """Activations of (step, layer), rows redrawn until the decision margin >= DELTA."""
    x = W.activations(cfg, step, layer)
    for t in range(x.shape[0]):
        att = 0
        while oracle.route_margin(oracle.router_logits(x[t:t + 1], wr), cfg) < DELTA:
            att += 1
            x[t] = W.activation_row(cfg, step, layer, t, att)
    return x


@pytest.mark.parametrize("cfg", [W.TINY, W.DECODE8_B32], ids=lambda c: c.name)
def test_router_gemv_and_routing(cfg):
    layers = list(range(min(cfg.L, 6)))
    xs = np.stack([_tie_free_x(cfg, 0, l, W.router_weights(cfg, l)) for l in layers])
    wrs = np.stack([W.router_weights(cfg, l) for l in layers])
    L, Tn = len(layers), xs.shape[1]
    p = E().route_params(cfg.mode, cfg.K, cfg.n_groups, cfg.topk_groups, cfg.scale, cfg.eps)
    idx = U.empty((L, Tn, cfg.K), "int32")
    w = U.empty((L, Tn, cfg.K))
    lo = U.empty((L, Tn, cfg.E))
    E().e0_route(p, L, Tn, cfg.E, None, False, U.f16(xs), U.f16(wrs), cfg.d, idx, w, lo)
    U.torch().cuda.synchronize()
    for i in range(L):
        rl = oracle.router_logits(xs[i], wrs[i])
        assert np.allclose(lo[i].cpu().numpy(), rl, rtol=1e-4, atol=1e-5)
        ridx, rw = oracle.route(rl, cfg)
        assert np.array_equal(idx[i].cpu().numpy(), ridx)
        assert np.abs(w[i].cpu().numpy() - rw).max() < 1e-5


def test_sigmoid_group_given_logits():
    cfg = W.DECODE8_B1
    rng = np.random.default_rng(7)
    rows = []
    while len(rows) < 300:
        r = rng.standard_normal((1, cfg.E)).astype(np.float32)
        if oracle.route_margin(r, cfg) >= DELTA:
            rows.append(r[0])
    lg = np.stack(rows)[None]
    p = E().route_params(1, cfg.K, cfg.n_groups, cfg.topk_groups, cfg.scale, cfg.eps)
    idx, w = _route_given(lg, p, fp16=False)
    ridx, rw = oracle.sigmoid_group(lg[0], cfg.K, cfg.n_groups, cfg.topk_groups, cfg.scale)
    assert np.array_equal(idx[0], ridx)
    assert np.abs(w[0] - rw).max() < 1e-6
    assert np.allclose(w[0].sum(1), cfg.scale, rtol=1e-6)
