"""GPU parity: the chained batch-1 decode (one token through stacked layers,
each layer's input the normed residual left by the one before) against the
fp64 oracle. Covers d_ff 256 / 512 / 1024, top-4 and top-8, ids out of range
or not resident, back-to-back calls on one workspace holding arbitrary bytes,
and the full 40-layer, 256-expert stack. Two bars, both rel-L2 <= 1e-3 on every
layer's output and residual: each layer against the oracle fed with the
residual the GPU produced before it, and the whole stack against the oracle's
own chain from the same input."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-3
EPS = 1e-6


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _inputs(cfg, L, step=0):
    lg = np.stack([W.given_logits(cfg, step, l)[0] for l in range(L)]).astype(np.float32)
    idx, w = oracle.softmax_topk(lg, cfg.K)
    r0 = W.residual0(cfg, step)
    g = np.stack([W.norm_weight(cfg, l) for l in range(L)])
    return idx.astype(np.int32), w.astype(np.float32), r0, g


def _pools(cfg, L, idx, slot_of=None):
    """Per layer: the experts it routes to (oracle format) and a slot table
    mapping them to 0..K-1 (-1 where the GPU table has the expert absent)."""
    mats, so = [], np.full((L, cfg.E), -1, dtype=np.int32)
    for l in range(L):
        for s, e in enumerate(int(v) for v in idx[l]):
            mats.append(gen.expert(cfg.seed, l, e if 0 <= e < cfg.E else 0, cfg.d, cfg.f))
            if 0 <= e < cfg.E and (slot_of is None or slot_of[l, e] >= 0):
                so[l, e] = s
    return mats, so


def _oracle(cfg, L, idx, w, r0, g, slot_of=None):
    """The oracle's own chain from r0 (free running)."""
    mats, so = _pools(cfg, L, idx, slot_of)
    return oracle.chain_decode(oracle.Experts(mats), cfg.K, so, cfg.E, cfg.d, cfg.f, r0.astype(np.float64), g,
                               EPS, idx, w.astype(np.float64))


def _check_forced(cfg, L, idx, w, r0, g, y, r, slot_of=None):
    """Each layer on its own: the oracle's layer l fed with the residual the
    GPU left after layer l - 1 (so the check does not depend on how the stack
    propagates earlier rounding)."""
    mats, so = _pools(cfg, L, idx, slot_of)
    yh, rh = y.cpu().numpy(), r.cpu().numpy()
    ey, er = [], []
    for l in range(L):
        rin = (r0 if l == 0 else rh[l - 1]).astype(np.float64)
        pool = oracle.Experts(mats[l * cfg.K:(l + 1) * cfg.K])
        yo, ro, _ = oracle.chain_decode(pool, cfg.K, so[l:l + 1], cfg.E, cfg.d, cfg.f, rin, g[l:l + 1], EPS,
                                        idx[l:l + 1], w[l:l + 1].astype(np.float64))
        ey.append(U.rel_l2(yh[l], yo[0]))
        er.append(U.rel_l2(rh[l], ro[0]))
    print("chain per layer (forced) y max %.2e r max %.2e" % (max(ey), max(er)))
    assert max(ey) <= TOL and max(er) <= TOL


def _run(cfg, L, store_stack, slot_of, idx, w, r0, g, ws=None):
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    if ws is None:
        ws = U.empty((E().workspace_bytes(E().E0_OP_CHAINED_DECODE, dims, L, 0, 0),), "uint8")
    y, r = U.empty((L, cfg.d)), U.empty((L, cfg.d))
    err = U.zeros((1,), "int32")
    E().e0_moe_chained_decode(dims, L, U.f32(r0), U.f16(g), EPS, U.i32(idx), U.f32(w), slot_of, cfg.E,
                              store_stack, y, r, ws, err)
    return y, r, err


def _check(y, r, yo, ro):
    yh, rh = y.cpu().numpy(), r.cpu().numpy()
    ey = [U.rel_l2(yh[l], yo[l]) for l in range(len(yo))]
    er = [U.rel_l2(rh[l], ro[l]) for l in range(len(ro))]
    print("chain (free) y", ["%.1e" % v for v in ey][-4:], "r", ["%.1e" % v for v in er][-4:])
    assert max(ey) <= TOL and max(er) <= TOL


def _setup(cfg, L):
    store = U.gpu_store(cfg, range(L))
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    st = E().stack_from_bundles(store, cfg.d, cfg.f, bb, cfg.E * bb)
    slot_of = U.i32(np.tile(np.arange(cfg.E, dtype=np.int32), (L, 1)))
    return store, st, slot_of


@pytest.mark.parametrize("K,f", [(4, 512), (8, 512), (4, 256), (4, 1024)])
def test_chain_matches_oracle(K, f):
    cfg = W.scaled(W.CHAIN35, E=24, K=K, f=f, L=4)
    L = cfg.L
    _store, st, slot_of = _setup(cfg, L)
    idx, w, r0, g = _inputs(cfg, L)
    y, r, err = _run(cfg, L, st, slot_of, idx, w, r0, g)
    U.torch().cuda.synchronize()
    assert int(err.item()) == 0
    yo, ro, oerr = _oracle(cfg, L, idx, w, r0, g)
    assert oerr == 0
    _check(y, r, yo, ro)
    _check_forced(cfg, L, idx, w, r0, g, y, r)


def test_chain_back_to_back_on_a_dirty_workspace():
    cfg = W.scaled(W.CHAIN35, E=24, L=3)
    L = cfg.L
    _store, st, slot_of = _setup(cfg, L)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    nbytes = E().workspace_bytes(E().E0_OP_CHAINED_DECODE, dims, L, 0, 0)
    ws = U.torch().from_numpy(np.random.default_rng(5).integers(0, 256, nbytes, dtype=np.uint8)).to(U.dev())
    runs = []
    for step in range(3):
        idx, w, r0, g = _inputs(cfg, L, step)
        runs.append((_run(cfg, L, st, slot_of, idx, w, r0, g, ws), (idx, w, r0, g)))
    U.torch().cuda.synchronize()
    for (y, r, err), (idx, w, r0, g) in runs:
        assert int(err.item()) == 0
        yo, ro, _ = _oracle(cfg, L, idx, w, r0, g)
        _check(y, r, yo, ro)


def test_chain_flags_and_skips_bad_experts():
    cfg = W.scaled(W.CHAIN35, E=24, L=2)
    L = cfg.L
    _store, st, _ = _setup(cfg, L)
    idx, w, r0, g = _inputs(cfg, L)
    idx = idx.copy()
    idx[0, 1] = 31  # out of range
    so = np.tile(np.arange(cfg.E, dtype=np.int32), (L, 1))
    so[1, idx[1, 2]] = -1  # not resident
    y, r, err = _run(cfg, L, st, U.i32(so), idx, w, r0, g)
    U.torch().cuda.synchronize()
    assert int(err.item()) == E().E0_DEV_BAD_ID | E().E0_DEV_NOT_RESIDENT
    yo, ro, oerr = _oracle(cfg, L, idx, w, r0, g, slot_of=so)
    assert oerr == 3
    _check(y, r, yo, ro)
    _check_forced(cfg, L, idx, w, r0, g, y, r, slot_of=so)


def test_chain35b_full_stack():
    cfg = W.CHAIN35
    L = cfg.L
    _store, st, slot_of = _setup(cfg, L)
    idx, w, r0, g = _inputs(cfg, L)
    y, r, err = _run(cfg, L, st, slot_of, idx, w, r0, g)
    U.torch().cuda.synchronize()
    assert int(err.item()) == 0
    _check_forced(cfg, L, idx, w, r0, g, y, r)
    yo, ro, _ = _oracle(cfg, L, idx, w, r0, g)
    _check(y, r, yo, ro)
