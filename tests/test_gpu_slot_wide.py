"""GPU parity of e0_slot_update at the width of its tables: 4096 experts
(the limit), 512 slots per layer, 16 tokens x K = 16 routed ids per layer
(repeats across tokens, as a batch has), two layers, five steps with the
ids in flight protected. slot_of and expert_of must equal the oracle's slot
rule replayed step by step, bit for bit, the copy counts its number of
placements, and every occupied slot must hold its expert's bundle."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def test_slot_update_4096_experts_512_slots():
    cfg = W.scaled(W.TINY, d=128, f=128, E=4096, K=16, L=2, B=16)
    L, B, K, Ex, S = cfg.L, cfg.B, cfg.K, cfg.E, 512
    T = U.torch()
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    store = U.gpu_store(cfg, range(L))
    pool = U.zeros((L, S, bb), "uint8")
    st_store = E().stack_from_bundles(store, cfg.d, cfg.f, bb, Ex * bb)
    st_pool = E().stack_from_bundles(pool, cfg.d, cfg.f, bb, S * bb)
    dims = E().moe_dims(cfg.d, cfg.f, Ex, K)
    slot_of = U.full((L, Ex), -1)
    expert_of = U.full((L, S), -1)
    err = U.zeros((1,), "int32")
    ncop = U.zeros((L,), "int32")
    ws = U.empty((E().workspace_bytes(E().E0_OP_SLOT_UPDATE, dims, L, B, S),), "uint8")
    so = np.full((L, Ex), -1, np.int32)
    eo = np.full((L, S), -1, np.int32)
    rng = np.random.default_rng(17)
    prev = None
    for t in range(5):
        # popular ids (a tenth of the experts) and rare ones: some stay resident, some change
        ids = np.where(rng.random((L, B, K)) < 0.6, rng.integers(0, Ex // 10, (L, B, K)),
                       rng.integers(0, Ex, (L, B, K))).astype(np.int32)
        E().e0_slot_update(dims, L, B, S, U.i32(ids), U.i32(prev) if prev is not None else None, slot_of, expert_of,
                           st_store, st_pool, ncop, ws, err)
        T.cuda.synchronize()
        assert int(err.item()) == 0
        nc = ncop.cpu().numpy()
        for l in range(L):
            rc, copies = oracle.slot_update(Ex, S, ids[l], prev[l] if prev is not None else [], so[l], eo[l])
            assert rc == 0 and nc[l] == len(copies), (t, l)
        assert np.array_equal(slot_of.cpu().numpy(), so) and np.array_equal(expert_of.cpu().numpy(), eo), t
        prev = ids
    ph, sh = pool.cpu().numpy(), store.cpu().numpy()
    for l in range(L):
        for s in range(S):
            if eo[l, s] >= 0:
                assert np.array_equal(ph[l, s], sh[l, eo[l, s]]), (l, s)
    print("occupied slots per layer", [(eo[l] >= 0).sum() for l in range(L)])
