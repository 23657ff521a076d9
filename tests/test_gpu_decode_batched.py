"""GPU parity of the batched (B > 1) staged decode at the 8B tier's expert shape
(d_model 2048, d_ff 512): a ragged number of sorted pairs (20, not a multiple of
the 16-pair h window the down kernel stages in LDS), experts holding 6, 4, 3, 2
and 1 tokens (gate/up token chunks of 4, 2 and 1, one with a padding slot), an
id out of range and an expert with no slot. Every token is checked against the
fp64 oracle's staged path, which skips the same contributions, and the device
error word must carry both bits."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-3
ELEM = 1e-4  # per token: max |y - ref| / max |ref|

# token -> its three routed experts; 99 is out of range, 13 has no slot
IDX = [[2, 5, 9], [2, 5, 13], [2, 7, 9], [2, 99, 5], [2, 11, 1], [2, 5, 0], [4, 7, 9]]
RESIDENT = [0, 1, 2, 4, 5, 7, 9, 11]


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def test_batched_decode_ragged_pairs_and_skips():
    cfg = W.scaled(W.DECODE8_B32, L=1, B=len(IDX), K=3, E=16)
    T = U.torch()
    d, f, Ex, K, B = cfg.d, cfg.f, cfg.E, cfg.K, cfg.B
    assert (d, f) == (2048, 512)
    bb = gen.bundle_bytes(d, f)
    S = len(RESIDENT)
    store = U.gpu_store(cfg, [0])
    pool = U.zeros((1, S, bb), "uint8")
    so = np.full(Ex, -1, np.int32)
    for s, e in enumerate(RESIDENT):
        pool[0, s].copy_(store[0, e])
        so[e] = s
    idx = np.array(IDX, np.int32)
    w = np.random.default_rng(11).uniform(0.1, 0.9, size=idx.shape).astype(np.float32)
    x = W.activations(cfg, 0, 0)
    dims = E().moe_dims(d, f, Ex, K)
    y = U.empty((1, B, d))
    err = U.zeros((1,), "int32")
    ws = U.empty((E().workspace_bytes(E().E0_OP_STAGED_DECODE, dims, 1, B, 0),), "uint8")
    E().e0_moe_staged_decode(dims, 1, B, U.f16(x[None]), U.i32(idx[None]), U.f32(w[None]), U.i32(so[None]), S,
                             E().stack_from_bundles(pool, d, f, bb, S * bb), None, y, ws, err)
    T.cuda.synchronize()
    assert int(err.item()) == E().E0_DEV_BAD_ID | E().E0_DEV_NOT_RESIDENT
    pool_list = [gen.expert(cfg.seed, 0, e, d, f) for e in RESIDENT]
    ref, rerr = oracle.moe_staged(oracle.Experts(pool_list), so, Ex, d, f, x, idx, w.astype(np.float64))
    assert rerr == 3
    got = y.cpu().numpy()[0]
    for t in range(B):
        U.assert_close(got[t], ref[t], TOL, ELEM, t)
