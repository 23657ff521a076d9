"""GPU parity: the slot update with the expert store in pinned host memory
(HBM slots as the cache of a host-DRAM store: koala.ai.kr walkthrough, Fig. 1
and the blocked-load discussion of Tab. 3; the store does not sit in the
accelerator's memory). At the 35B bundle size the tables after every update
equal the oracle's slot rule replayed on the same routing, bit for bit, and
every resident slot holds the CPU generator's bytes of its expert; at the
tiny shape the pool and tables also equal those of the same update from a
device-memory store. A store in host memory the device cannot reach is
refused before anything is enqueued."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _update(cfg, L, S, store_t, steps):
    T = U.torch()
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    store = E().stack_from_bundles(store_t, cfg.d, cfg.f, bb, cfg.E * bb)
    pool_t = U.zeros((L, S, bb), "uint8")
    pool = E().stack_from_bundles(pool_t, cfg.d, cfg.f, bb, S * bb)
    slot_of = U.full((L, cfg.E), -1)
    expert_of = U.full((L, S), -1)
    ws = U.empty((E().workspace_bytes(E().E0_OP_SLOT_UPDATE, dims, L, cfg.B, S),), "uint8")
    err = U.zeros((1,), "int32")
    n_copied = U.zeros((L,), "int32")
    prev = None
    copied = 0
    for ids in steps:
        cur = U.i32(ids)
        E().e0_slot_update(dims, L, cfg.B, S, cur, prev, slot_of, expert_of, store, pool, n_copied, ws, err)
        T.cuda.synchronize()
        copied += int(n_copied.sum().item())
        prev = cur
    assert int(err.item()) == 0
    return pool_t.cpu().numpy(), slot_of.cpu().numpy(), expert_of.cpu().numpy(), copied


def _steps(cfg, L, n, seed=3):
    rng = np.random.default_rng(seed)
    return [np.stack([np.stack([rng.permutation(cfg.E)[:cfg.K] for _ in range(cfg.B)]) for _ in range(L)])
            .astype(np.int32) for _ in range(n)]


def test_host_store_update_equals_device_store_update():
    T = U.torch()
    cfg = W.scaled(W.TINY, L=2, B=2)
    L, S = 2, 16
    dev_store = U.gpu_store(cfg, range(L))
    host_store = T.empty(dev_store.shape, dtype=T.uint8, pin_memory=True)
    host_store.copy_(dev_store)
    T.cuda.synchronize()
    steps = _steps(cfg, L, 4)
    pd, sd, ed, nd = _update(cfg, L, S, dev_store, steps)
    ph, sh, eh, nh = _update(cfg, L, S, host_store, steps)
    assert nd == nh and nd > 0
    assert np.array_equal(sd, sh) and np.array_equal(ed, eh)
    assert np.array_equal(pd, ph)
    st = host_store.numpy()
    for l in range(L):
        for s in range(S):
            if eh[l, s] >= 0:
                assert np.array_equal(ph[l, s], st[l, eh[l, s]])


def test_unmapped_host_store_is_refused():
    T = U.torch()
    cfg = W.scaled(W.TINY, L=1, B=1)
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    plain = np.zeros((1, cfg.E, bb + 16), dtype=np.uint8)  # ordinary pageable host memory
    base = plain.ctypes.data
    off = (-base) % 16
    arr = T.from_numpy(plain.reshape(-1)[off:off + cfg.E * bb].reshape(1, cfg.E, bb))
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    store = E().stack_from_bundles(arr, cfg.d, cfg.f, bb, cfg.E * bb)
    pool_t = U.zeros((1, 8, bb), "uint8")
    pool = E().stack_from_bundles(pool_t, cfg.d, cfg.f, bb, 8 * bb)
    ws = U.empty((E().workspace_bytes(E().E0_OP_SLOT_UPDATE, dims, 1, 1, 8),), "uint8")
    err = U.zeros((1,), "int32")
    # The requested experts are already resident, so even an accepted call
    # would copy nothing and never read the store.
    so = np.full((1, cfg.E), -1, np.int32)
    so[0, [1, 2, 3, 4]] = [0, 1, 2, 3]
    eo = np.full((1, 8), -1, np.int32)
    eo[0, :4] = [1, 2, 3, 4]
    with pytest.raises(E().E0Error) as ei:
        E().e0_slot_update(dims, 1, 1, 8, U.i32([[[1, 2, 3, 4]]]), None, U.i32(so), U.i32(eo), store, pool, None, ws,
                           err)
    assert ei.value.status == E().E0_ERR_INVALID_ARG
    T.cuda.synchronize()
    assert int(err.item()) == 0


def test_host_store_35b_bundles_follow_the_oracle_rule():
    T = U.torch()
    cfg = W.DECODE35
    L, S, K, steps = 2, cfg.S, cfg.K, 6
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    # The store filled on the CPU from the generator, in pinned host memory.
    host = T.empty((L, cfg.E, bb), dtype=T.uint8, pin_memory=True)
    hn = host.numpy()
    for l in range(L):
        hn[l] = gen.layer_store(cfg.seed, l, cfg.E, cfg.d, cfg.f)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, K)
    store = E().stack_from_bundles(host, cfg.d, cfg.f, bb, cfg.E * bb)
    pool_t = U.zeros((L, S, bb), "uint8")
    pool = E().stack_from_bundles(pool_t, cfg.d, cfg.f, bb, S * bb)
    slot_of = U.full((L, cfg.E), -1)
    expert_of = U.full((L, S), -1)
    ws = U.empty((E().workspace_bytes(E().E0_OP_SLOT_UPDATE, dims, L, 1, S),), "uint8")
    err = U.zeros((1,), "int32")
    n_copied = U.zeros((L,), "int32")
    so = np.full((L, cfg.E), -1, np.int32)
    eo = np.full((L, S), -1, np.int32)
    prev, prev_ids, total = None, None, 0
    for t in range(steps):
        ids = np.stack([oracle.softmax_topk(W.given_logits(cfg, t, l).astype(np.float32), K)[0][0] for l in range(L)])
        cur = U.i32(ids[:, None, :])
        E().e0_slot_update(dims, L, 1, S, cur, prev, slot_of, expert_of, store, pool, n_copied, ws, err)
        T.cuda.synchronize()
        n = 0
        for l in range(L):
            rc, copies = oracle.slot_update(cfg.E, S, ids[l], prev_ids[l] if t else [], so[l], eo[l])
            assert rc == 0
            n += len(copies)
        assert np.array_equal(slot_of.cpu().numpy(), so) and np.array_equal(expert_of.cpu().numpy(), eo), t
        assert int(n_copied.sum().item()) == n
        total += n
        pl = pool_t.cpu().numpy()
        for l in range(L):
            for s_ in range(S):
                if eo[l, s_] >= 0:
                    assert np.array_equal(pl[l, s_], hn[l, eo[l, s_]]), (t, l, s_)
        prev, prev_ids = cur, ids
    assert int(err.item()) == 0
    print("host-store slot updates, experts copied over the host link:", total)
