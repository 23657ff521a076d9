"""GPU parity: slot update (tables bit-exact, pool bytes equal to the store)
and staged decode (rel-L2 <= 1e-3 against the fp64 oracle), at the tiny shape
and at the 35B-tier shape through 40 layers."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-3
ELEM = 1e-4  # per token: max |y - ref| / max |ref| (fp32 accumulation of exact weights: ~1e-6)


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _stacks(store, pool, cfg):
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    return (E().stack_from_bundles(store, cfg.d, cfg.f, bb, store.shape[1] * bb),
            E().stack_from_bundles(pool, cfg.d, cfg.f, bb, pool.shape[1] * bb))


def _replay_tables(cfg, L, S, routes):
    """Oracle slot rule over a sequence of routings [steps][L][B][K]."""
    so = np.full((L, cfg.E), -1, np.int32)
    eo = np.full((L, S), -1, np.int32)
    out = []
    for t, r in enumerate(routes):
        for l in range(L):
            cur = routes[t - 1][l] if t > 0 else []
            rc, _ = oracle.slot_update(cfg.E, S, r[l], cur, so[l], eo[l])
            assert rc == 0
        out.append((so.copy(), eo.copy()))
    return out


def _run_steps(cfg, L, steps, S, logits_fn, x_fn, overlap=True, hot_set=False):
    """Route -> slot update -> decode for `steps` steps; returns per-step
    (idx, w, y, slot_of, expert_of) on the host plus the device store/pool."""
    from int4_gather_swiglu_amd.pipeline import StagedPipeline
    T = U.torch()
    store = U.gpu_store(cfg, range(L))
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    pool = U.zeros((L, S, bb), "uint8")
    st_store, st_pool = _stacks(store, pool, cfg)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    pipe = StagedPipeline(dims, L, cfg.B, S, st_store, st_pool, side_stream=overlap, hot_set=hot_set)
    p = E().route_params(cfg.mode, cfg.K, cfg.n_groups, cfg.topk_groups, cfg.scale, cfg.eps)
    lgs = [U.f16(logits_fn(t)) for t in range(steps)]
    xs = [U.f16(x_fn(t)) for t in range(steps)]
    ys = [U.empty((L, cfg.B, cfg.d)) for _ in range(steps)]
    recs = []
    pipe.route_given(0, p, lgs[0])
    pipe.update(0, None)
    pipe.join()
    for t in range(steps):
        if t + 1 < steps:
            pipe.route_given((t + 1) % 2, p, lgs[t + 1])
            idx_next = pipe.idx[(t + 1) % 2]
        # snapshot the tables step t decodes with (the side stream may change them)
        T.cuda.current_stream().synchronize()
        pipe.side.synchronize()
        rec = dict(idx=pipe.idx[t % 2].cpu().numpy(), w=pipe.w[t % 2].cpu().numpy(),
                   slot_of=pipe.slot_of.cpu().numpy(), expert_of=pipe.expert_of.cpu().numpy(),
                   last_use=pipe.last_use.cpu().numpy())
        if t + 1 < steps:
            pipe.update((t + 1) % 2, t % 2)
        pipe.decode(t % 2, xs[t], ys[t])
        if t + 1 < steps:
            pipe.join()
        recs.append(rec)
    T.cuda.synchronize()
    for t in range(steps):
        recs[t]["y"] = ys[t].cpu().numpy()
    assert int(pipe.err.item()) == 0
    return recs, store, pool


def _check_layer(cfg, layer, rec, x, tol=TOL):
    ids = sorted(set(rec["idx"][layer].ravel().tolist()))
    experts = {e: gen.expert(cfg.seed, layer, e, cfg.d, cfg.f) for e in ids}
    lst = [experts.get(e, experts[ids[0]]) for e in range(cfg.E)]
    ref, err = oracle.moe_exact(oracle.Experts(lst), cfg.d, cfg.f, x, rec["idx"][layer], rec["w"][layer].astype(np.float64))
    assert err == 0
    r, _ = U.assert_close(rec["y"][layer], ref, tol, ELEM, (cfg.name, layer))
    return r


@pytest.mark.parametrize("B", [1, 3, 8])
def test_tiny_decode_steps(B):
    cfg = W.scaled(W.TINY, B=B, L=2, S=2 * B * 4)
    L, steps, S = cfg.L, 4, min(cfg.E, 2 * B * cfg.K)
    recs, store, pool = _run_steps(cfg, L, steps, S, lambda t: np.stack([W.given_logits(cfg, t, l) for l in range(L)]),
                                   lambda t: np.stack([W.activations(cfg, t, l) for l in range(L)]))
    routes = [r["idx"] for r in recs]
    for t in range(steps):
        ridx, _ = oracle.softmax_topk(np.stack([W.given_logits(cfg, t, l) for l in range(L)]).reshape(-1, cfg.E)
                                      .astype(np.float32), cfg.K)
        assert np.array_equal(recs[t]["idx"].reshape(-1, cfg.K), ridx)
    tables = _replay_tables(cfg, L, S, routes)
    for t in range(steps):
        assert np.array_equal(recs[t]["slot_of"], tables[t][0]), t
        assert np.array_equal(recs[t]["expert_of"], tables[t][1]), t
        for l in range(L):
            _check_layer(cfg, l, recs[t], W.activations(cfg, t, l))


def test_hot_set_decode_steps():
    # The pool as a least-recently-used hot set (S between one step's need and
    # the store): tables step by step as the oracle's rule, and every layer's
    # output exact whatever the policy evicted.
    from oracle import lru as R
    cfg = W.scaled(W.TINY, B=2, L=2, E=32, S=20)
    L, steps, S = cfg.L, 6, 20
    recs, store, pool = _run_steps(cfg, L, steps, S, lambda t: np.stack([W.given_logits(cfg, t, l) for l in range(L)]),
                                   lambda t: np.stack([W.activations(cfg, t, l) for l in range(L)]), hot_set=True)
    so = [[-1] * cfg.E for _ in range(L)]
    eo = [[-1] * S for _ in range(L)]
    lu = [[-1] * S for _ in range(L)]
    for t in range(steps):
        for l in range(L):
            prev = recs[t - 1]["idx"][l].ravel().tolist() if t > 0 else []
            _, bad = R.slot_update_lru(cfg.E, S, recs[t]["idx"][l].ravel().tolist(), prev, so[l], eo[l], lu[l], t)
            assert not bad
        assert np.array_equal(recs[t]["slot_of"], np.array(so)), t
        assert np.array_equal(recs[t]["expert_of"], np.array(eo)), t
        assert np.array_equal(recs[t]["last_use"], np.array(lu)), t
        for l in range(L):
            _check_layer(cfg, l, recs[t], W.activations(cfg, t, l))


def test_pool_bytes_equal_store_after_update():
    cfg = W.scaled(W.TINY, L=2, B=2)
    S = 16
    recs, store, pool = _run_steps(cfg, 2, 3, S, lambda t: np.stack([W.given_logits(cfg, t, l) for l in range(2)]),
                                   lambda t: np.stack([W.activations(cfg, t, l) for l in range(2)]))
    st = store.cpu().numpy()
    pl = pool.cpu().numpy()
    eo = recs[-1]["expert_of"]  # tables before the last step's decode = final tables
    for l in range(2):
        for s in range(S):
            if eo[l, s] >= 0:
                assert np.array_equal(pl[l, s], st[l, eo[l, s]])


def test_overlap_matches_single_stream():
    cfg = W.scaled(W.TINY, L=3, B=2)
    S = 16
    args = (cfg, 3, 5, S, lambda t: np.stack([W.given_logits(cfg, t, l) for l in range(3)]),
            lambda t: np.stack([W.activations(cfg, t, l) for l in range(3)]))
    a, _, _ = _run_steps(*args, overlap=True)
    b, _, _ = _run_steps(*args, overlap=False)
    for ra, rb in zip(a, b):
        assert np.array_equal(ra["y"], rb["y"])


def test_decode35b_full_shape_sampled():
    cfg = W.DECODE35
    L, steps, S = cfg.L, 3, cfg.S
    recs, store, pool = _run_steps(cfg, L, steps, S,
                                   lambda t: np.stack([W.given_logits(cfg, t, l) for l in range(L)]),
                                   lambda t: np.stack([W.activations(cfg, t, l) for l in range(L)]))
    routes = [r["idx"] for r in recs]
    tables = _replay_tables(cfg, L, S, routes)
    rs = []
    for t in range(steps):
        assert np.array_equal(recs[t]["slot_of"], tables[t][0])
        assert np.array_equal(recs[t]["expert_of"], tables[t][1])
        for l in (0, 17, 39) if t < 2 else (5,):
            rs.append(_check_layer(cfg, l, recs[t], W.activations(cfg, t, l)))
    print("decode35b rel-L2 max", max(rs))


def test_device_errors_flag_and_skip():
    cfg = W.scaled(W.TINY, L=1, B=1)
    T = U.torch()
    L, S = 1, 8
    store = U.gpu_store(cfg, [0])
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    pool = U.zeros((L, S, bb), "uint8")
    st_store, st_pool = _stacks(store, pool, cfg)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    idx = U.i32([[[3, 5, 9, 11]]])
    w = U.f32([[[0.4, 0.3, 0.2, 0.1]]])
    slot_of = U.full((1, cfg.E), -1)
    expert_of = U.full((1, S), -1)
    err = U.zeros((1,), "int32")
    ws = U.empty((E().workspace_bytes(E().E0_OP_SLOT_UPDATE, dims, 1, 1, S),), "uint8")
    E().e0_slot_update(dims, 1, 1, S, U.i32([[[3, 5, 9, 1]]]), None, slot_of, expert_of, st_store, st_pool, None, ws, err)
    x = W.activations(cfg, 0, 0)[:1]
    y = U.empty((1, 1, cfg.d))
    wsd = U.empty((E().workspace_bytes(E().E0_OP_STAGED_DECODE, dims, 1, 1, 0),), "uint8")
    E().e0_moe_staged_decode(dims, 1, 1, U.f16(x[None]), idx, w, slot_of, S, st_pool, None, y, wsd, err)
    T.cuda.synchronize()
    assert int(err.item()) == E().E0_DEV_NOT_RESIDENT  # expert 11 has no slot
    # the oracle's staged path skips the same contribution
    so = slot_of.cpu().numpy()[0]
    eo = expert_of.cpu().numpy()[0]
    experts = [gen.expert(cfg.seed, 0, e, cfg.d, cfg.f) for e in range(cfg.E)]
    pool_list = [experts[e] if e >= 0 else experts[0] for e in eo]
    ref, rerr = oracle.moe_staged(oracle.Experts(pool_list), so, cfg.E, cfg.d, cfg.f, x, np.array([[3, 5, 9, 11]]),
                                  np.array([[0.4, 0.3, 0.2, 0.1]], dtype=np.float32).astype(np.float64))
    assert rerr == 2
    assert U.rel_l2(y.cpu().numpy()[0], ref) <= TOL
    # an id out of range
    err.zero_()
    E().e0_moe_staged_decode(dims, 1, 1, U.f16(x[None]), U.i32([[[3, 5, 9, 16]]]), w, slot_of, S, st_pool, None, y,
                             wsd, err)
    T.cuda.synchronize()
    assert int(err.item()) == E().E0_DEV_BAD_ID


def test_slot_update_no_free_slot_places_what_fits():
    cfg = W.scaled(W.TINY, L=1, B=1)
    T = U.torch()
    S = 4
    store = U.gpu_store(cfg, [0])
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    pool = U.zeros((1, S, bb), "uint8")
    st_store, st_pool = _stacks(store, pool, cfg)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    slot_of = U.full((1, cfg.E), -1)
    expert_of = U.full((1, S), -1)
    err = U.zeros((1,), "int32")
    ws = U.empty((E().workspace_bytes(E().E0_OP_SLOT_UPDATE, dims, 1, 1, S),), "uint8")
    ncop = U.zeros((1,), "int32")
    E().e0_slot_update(dims, 1, 1, S, U.i32([[[0, 2, 4, 6]]]), None, slot_of, expert_of, st_store, st_pool, ncop, ws, err)
    E().e0_slot_update(dims, 1, 1, S, U.i32([[[1, 3, 5, 7]]]), U.i32([[[6, 4, 0, 9]]]), slot_of, expert_of,
                       st_store, st_pool, ncop, ws, err)
    T.cuda.synchronize()
    so = np.full(cfg.E, -1, np.int32)
    eo = np.full(S, -1, np.int32)
    oracle.slot_update(cfg.E, S, [0, 2, 4, 6], [], so, eo)
    rc, copies = oracle.slot_update(cfg.E, S, [1, 3, 5, 7], [6, 4, 0, 9], so, eo)
    assert rc == 4 and int(err.item()) == E().E0_DEV_NO_SLOT
    assert np.array_equal(slot_of.cpu().numpy()[0], so) and np.array_equal(expert_of.cpu().numpy()[0], eo)
    assert int(ncop.item()) == len(copies) == 1
