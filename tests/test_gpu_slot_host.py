"""GPU parity: the slot update with the expert store in pinned host memory
(HBM slots as the cache of a host-DRAM store). The pool bytes and both slot
tables must equal, bit for bit, those of the same update from a device-memory
store; a store in host memory the device cannot reach is refused before
anything is enqueued."""
import numpy as np
import pytest

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
