"""GPU parity: e0_slot_update_lru (the slot pool as a per-layer least-recently-
used hot set of the store) against the oracle's rule (oracle/lru.py), step by
step over skewed routing sequences: slot_of, expert_of, last_use and the copy
counts bit-exact after every step, every resident slot's bytes equal to its
expert's bundle in the store, and the hit rate above the plain lowest-slot
rule's on the same sequence. Covers batch 1 and 4, pools from one step's
worth to half the store, and the validation of the extra arguments."""
import numpy as np
import pytest

from e0inputs import gen, workloads as W
from oracle import lru as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _steps(E_, K, B, L, n, seed):
    """Skewed routing: most picks from a small popular subset that drifts."""
    rng = np.random.default_rng(seed)
    out = []
    for t in range(n):
        hot = (np.arange(E_ // 4) + t // 8) % E_
        ids = np.empty((L, B, K), dtype=np.int32)
        for l in range(L):
            for b in range(B):
                pick = rng.choice(hot, K, replace=False) if rng.random() < 0.8 else rng.choice(E_, K, replace=False)
                ids[l, b] = pick
        out.append(ids)
    return out


def _run(cfg, L, S, steps, lru=True):
    T = U.torch()
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    store_t = U.gpu_store(cfg, range(L))
    store = E().stack_from_bundles(store_t, cfg.d, cfg.f, bb, cfg.E * bb)
    pool_t = U.zeros((L, S, bb), "uint8")
    pool = E().stack_from_bundles(pool_t, cfg.d, cfg.f, bb, S * bb)
    slot_of, expert_of, last_use = U.full((L, cfg.E), -1), U.full((L, S), -1), U.full((L, S), -1)
    ws = U.empty((E().workspace_bytes(E().E0_OP_SLOT_UPDATE, dims, L, cfg.B, S),), "uint8")
    err, n_copied = U.zeros((1,), "int32"), U.zeros((L,), "int32")
    # oracle state
    oso = [[-1] * cfg.E for _ in range(L)]
    oeo = [[-1] * S for _ in range(L)]
    olu = [[-1] * S for _ in range(L)]
    prev, prev_np = None, None
    copies = 0
    for t, ids in enumerate(steps):
        cur = U.i32(ids)
        if lru:
            E().e0_slot_update_lru(dims, L, cfg.B, S, cur, prev, slot_of, expert_of, last_use, t, store, pool,
                                   n_copied, ws, err)
        else:
            E().e0_slot_update(dims, L, cfg.B, S, cur, prev, slot_of, expert_of, store, pool, n_copied, ws, err)
        T.cuda.synchronize()
        nc = n_copied.cpu().numpy()
        copies += int(nc.sum())
        if lru:
            for l in range(L):
                keep = [] if prev_np is None else prev_np[l].ravel().tolist()
                cp, bad = R.slot_update_lru(cfg.E, S, ids[l].ravel().tolist(), keep, oso[l], oeo[l], olu[l], t)
                assert not bad
                assert nc[l] == len(cp), (t, l)
            assert np.array_equal(slot_of.cpu().numpy(), np.array(oso)), t
            assert np.array_equal(expert_of.cpu().numpy(), np.array(oeo)), t
            assert np.array_equal(last_use.cpu().numpy(), np.array(olu)), t
        prev, prev_np = cur, ids
    assert int(err.item()) == 0
    pool_np, store_np, eo = pool_t.cpu().numpy(), store_t.cpu().numpy(), expert_of.cpu().numpy()
    for l in range(L):
        for s in range(S):
            if eo[l, s] >= 0:
                assert np.array_equal(pool_np[l, s], store_np[l, eo[l, s]]), (l, s)
    return copies


@pytest.mark.parametrize("B,S", [(1, 8), (1, 24), (4, 48), (1, 64)])
def test_lru_matches_oracle_and_beats_lowest_slot(B, S):
    cfg = W.scaled(W.DECODE35, L=2, B=B, E=128, K=4, S=S)
    steps = _steps(cfg.E, cfg.K, B, 2, 40, seed=B * 100 + S)
    c_lru = _run(cfg, 2, S, steps, lru=True)
    c_low = _run(cfg, 2, S, steps, lru=False)
    print(f"B={B} S={S}: copies over 40 steps, LRU {c_lru} vs lowest slot {c_low}")
    if S > 2 * cfg.K * B:
        assert c_lru <= c_low


def test_lru_validation():
    cfg = W.scaled(W.DECODE35, L=1, B=1, E=16, K=4, S=8)
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    store_t = U.zeros((cfg.E, bb), "uint8")
    pool_t = U.zeros((8, bb), "uint8")
    st = E().stack_from_bundles(store_t, cfg.d, cfg.f, bb, bb)
    po = E().stack_from_bundles(pool_t, cfg.d, cfg.f, bb, bb)
    ids = U.i32(np.arange(4, dtype=np.int32).reshape(1, 1, 4))
    so, eo, lu = U.full((1, cfg.E), -1), U.full((1, 8), -1), U.full((1, 8), -1)
    ws = U.empty((E().workspace_bytes(E().E0_OP_SLOT_UPDATE, dims, 1, 1, 8),), "uint8")
    err, nc = U.zeros((1,), "int32"), U.zeros((1,), "int32")
    with pytest.raises(E().E0Error):
        E().e0_slot_update_lru(dims, 1, 1, 8, ids, None, so, eo, None, 0, st, po, nc, ws, err)
    with pytest.raises(E().E0Error):
        E().e0_slot_update_lru(dims, 1, 1, 8, ids, None, so, eo, lu, -1, st, po, nc, ws, err)
