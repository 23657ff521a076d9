"""GPU parity: the 8B-tier decode with sigmoid-group routing (8 groups, keep
4 by top-2 sum, scale 2.5, K=8) from each layer's own router, at batch 1 and
batch 32 (distinct tokens, deduplicated experts), through 24 layers.
Routing bit-exact (inputs redrawn until every decision has margin >= 1e-3),
slot tables bit-exact, outputs rel-L2 <= 1e-3 on sampled layers/tokens."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-3
ELEM = 1e-4  # per token: max |y - ref| / max |ref|
DELTA = 1e-3


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _tie_free(cfg, t, l, wr):
    x = W.activations(cfg, t, l)
    for i in range(x.shape[0]):
        att = 0
        while oracle.route_margin(oracle.router_logits(x[i:i + 1], wr), cfg) < DELTA:
            att += 1
            x[i] = W.activation_row(cfg, t, l, i, att)
    return x


@pytest.mark.parametrize("cfg", [W.DECODE8_B1, W.DECODE8_B32], ids=lambda c: c.name)
def test_decode8b_steps(cfg):
    from int4_gather_swiglu_amd.pipeline import StagedPipeline
    T = U.torch()
    L, B, K, S, steps = cfg.L, cfg.B, cfg.K, cfg.S, 3
    wr_h = np.stack([W.router_weights(cfg, l) for l in range(L)])
    xs_h = [np.stack([_tie_free(cfg, t, l, wr_h[l]) for l in range(L)]) for t in range(steps)]
    store = U.gpu_store(cfg, range(L))
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    pool = U.zeros((L, S, bb), "uint8")
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, K)
    pipe = StagedPipeline(dims, L, B, S, E().stack_from_bundles(store, cfg.d, cfg.f, bb, cfg.E * bb),
                          E().stack_from_bundles(pool, cfg.d, cfg.f, bb, S * bb))
    p = E().route_params(1, K, cfg.n_groups, cfg.topk_groups, cfg.scale, cfg.eps)
    wr = U.f16(wr_h)
    xs = [U.f16(x) for x in xs_h]
    lo = U.empty((L, B, cfg.E))
    ys = [U.empty((L, B, cfg.d)) for _ in range(steps)]
    recs = []
    pipe.route_router(0, p, xs[0], wr, lo)
    pipe.update(0, None)
    pipe.join()
    for t in range(steps):
        if t + 1 < steps:
            pipe.route_router((t + 1) % 2, p, xs[t + 1], wr, lo)
        T.cuda.synchronize()
        recs.append(dict(idx=pipe.idx[t % 2].cpu().numpy(), w=pipe.w[t % 2].cpu().numpy(),
                         slot_of=pipe.slot_of.cpu().numpy(), expert_of=pipe.expert_of.cpu().numpy()))
        if t + 1 < steps:
            pipe.update((t + 1) % 2, t % 2)
        pipe.decode(t % 2, xs[t], ys[t])
        if t + 1 < steps:
            pipe.join()
    T.cuda.synchronize()
    assert int(pipe.err.item()) == 0
    so = np.full((L, cfg.E), -1, np.int32)
    eo = np.full((L, S), -1, np.int32)
    rs = []
    for t in range(steps):
        for l in range(L):
            ridx, rw = oracle.route(oracle.router_logits(xs_h[t][l], wr_h[l]), cfg)
            assert np.array_equal(recs[t]["idx"][l], ridx), (t, l)
            assert np.abs(recs[t]["w"][l] - rw).max() < 1e-5
            rc, _ = oracle.slot_update(cfg.E, S, ridx, recs[t - 1]["idx"][l] if t > 0 else [], so[l], eo[l])
            assert rc == 0
        assert np.array_equal(recs[t]["slot_of"], so) and np.array_equal(recs[t]["expert_of"], eo)
        y = ys[t].cpu().numpy()
        for l in ((0, 23) if t == 0 else (11,)):
            tok = np.arange(B) if B <= 4 else np.array([0, 7, 19, 31])
            ids = sorted(set(recs[t]["idx"][l][tok].ravel().tolist()))
            mats = {e: gen.expert(cfg.seed, l, e, cfg.d, cfg.f) for e in ids}
            lst = [mats.get(e, mats[ids[0]]) for e in range(cfg.E)]
            ref, _ = oracle.moe_exact(oracle.Experts(lst), cfg.d, cfg.f, xs_h[t][l][tok], recs[t]["idx"][l][tok],
                                      recs[t]["w"][l][tok].astype(np.float64))
            rs.append(U.assert_close(y[l][tok], ref, TOL, ELEM, (t, l))[0])
    uniq = [len(set(recs[0]["idx"][l].ravel().tolist())) for l in range(L)]
    print(cfg.name, "rel-L2", max(rs), "unique experts/layer", min(uniq), max(uniq))
    assert max(rs) <= TOL
