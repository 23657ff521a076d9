"""GPU parity of e0_moe_staged_decode_noalloc (the staged decode with the
library's own fixed workspace, for callers that cannot allocate) against
e0_moe_staged_decode with a caller workspace, through the C ABI: two calls in
a row, the second smaller (35B-tier shape, 8 layers at batch 1 on the
single-launch kernel; then the tiny shape, 2 layers at batch 3 on the batched
kernels). Outputs must equal the existing entry point's bit for bit (same
kernels, fixed summation order) and the oracle's within rel-L2 1e-3 and the
decode's per-element bound; the device error word stays clear."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-3
ELEM = 1e-4


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _case(cfg, L):
    """Store, pool filled by the slot update for one step's routing, and the inputs."""
    T = U.torch()
    S = min(cfg.E, 2 * cfg.B * cfg.K)
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    store = U.gpu_store(cfg, range(L))
    pool = U.zeros((L, S, bb), "uint8")
    st_store = E().stack_from_bundles(store, cfg.d, cfg.f, bb, cfg.E * bb)
    st_pool = E().stack_from_bundles(pool, cfg.d, cfg.f, bb, S * bb)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    lg = np.stack([W.given_logits(cfg, 0, l) for l in range(L)]).reshape(L * cfg.B, cfg.E).astype(np.float32)
    idx, w = oracle.softmax_topk(lg, cfg.K)
    idx = idx.reshape(L, cfg.B, cfg.K)
    w = w.astype(np.float32).reshape(L, cfg.B, cfg.K)
    x = np.stack([W.activations(cfg, 0, l) for l in range(L)])
    slot_of = U.full((L, cfg.E), -1)
    expert_of = U.full((L, S), -1)
    err = U.zeros((1,), "int32")
    ws = U.empty((E().workspace_bytes(E().E0_OP_SLOT_UPDATE, dims, L, cfg.B, S),), "uint8")
    E().e0_slot_update(dims, L, cfg.B, S, U.i32(idx), None, slot_of, expert_of, st_store, st_pool, None, ws, err)
    T.cuda.synchronize()
    assert int(err.item()) == 0
    return dict(dims=dims, S=S, st_pool=st_pool, slot_of=slot_of, idx=idx, w=w, x=x, store=store, pool=pool)


def _both(cfg, L, c):
    T = U.torch()
    xd, idd, wd = U.f16(c["x"]), U.i32(c["idx"]), U.f32(c["w"])
    y_ref = U.full((L, cfg.B, cfg.d), float("nan"), "float32")
    y_na = U.full((L, cfg.B, cfg.d), float("nan"), "float32")
    err = U.zeros((1,), "int32")
    ws = U.empty((E().workspace_bytes(E().E0_OP_STAGED_DECODE, c["dims"], L, cfg.B, 0),), "uint8")
    E().e0_moe_staged_decode(c["dims"], L, cfg.B, xd, idd, wd, c["slot_of"], c["S"], c["st_pool"], None, y_ref, ws,
                             err)
    E().e0_moe_staged_decode_noalloc(c["dims"], L, cfg.B, xd, idd, wd, c["slot_of"], c["S"], c["st_pool"], None,
                                     y_na, err)
    T.cuda.synchronize()
    assert int(err.item()) == 0
    a, b = y_ref.cpu().numpy(), y_na.cpu().numpy()
    assert np.array_equal(a, b), float(np.nanmax(np.abs(a - b)))
    for l in range(L):
        ids = sorted(set(c["idx"][l].ravel().tolist()))
        mats = {e: gen.expert(cfg.seed, l, e, cfg.d, cfg.f) for e in ids}
        lst = [mats.get(e, mats[ids[0]]) for e in range(cfg.E)]
        ref, rerr = oracle.moe_exact(oracle.Experts(lst), cfg.d, cfg.f, c["x"][l], c["idx"][l],
                                     c["w"][l].astype(np.float64))
        assert rerr == 0
        U.assert_close(b[l], ref, TOL, ELEM, l)


def test_noalloc_matches_workspace_decode_two_calls():
    big = W.DECODE35
    _both(big, 8, _case(big, 8))
    small = W.scaled(W.TINY, B=3)
    _both(small, 2, _case(small, 2))
