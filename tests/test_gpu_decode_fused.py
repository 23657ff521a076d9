"""GPU parity: the batch-1 staged decode at d_model 2048, which runs as one
launch (gate/up items hand their h to down items through in-launch flags).
Covers d_ff 256 / 512 / 1024, top-4 and top-8, the shared expert with its
unmerged LoRA, ids out of range or not resident, back-to-back calls on one
workspace, and a workspace holding arbitrary bytes before the first call.
Outputs rel-L2 <= 1e-3 against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-3
ELEM = 1e-4  # per token: max |y - ref| / max |ref|


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _setup(cfg, L):
    store = U.gpu_store(cfg, range(L))
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    st = E().stack_from_bundles(store, cfg.d, cfg.f, bb, cfg.E * bb)
    slot_of = U.i32(np.tile(np.arange(cfg.E, dtype=np.int32), (L, 1)))
    return store, st, slot_of


def _routing(cfg, L, step):
    lg = np.stack([W.given_logits(cfg, step, l) for l in range(L)]).reshape(L, cfg.E).astype(np.float32)
    idx, w = oracle.softmax_topk(lg, cfg.K)
    return idx.reshape(L, 1, cfg.K).astype(np.int32), w.reshape(L, 1, cfg.K).astype(np.float32)


def _ref_layer(cfg, l, x, idx, w):
    ids = sorted(set(int(e) for e in idx.ravel() if 0 <= e < cfg.E))
    mats = {e: gen.expert(cfg.seed, l, e, cfg.d, cfg.f) for e in ids}
    lst = [mats.get(e, mats[ids[0]]) for e in range(cfg.E)]
    ref, _ = oracle.moe_exact(oracle.Experts(lst), cfg.d, cfg.f, x[None], idx[None], w[None].astype(np.float64))
    return ref[0]


@pytest.mark.parametrize("K,f", [(4, 512), (8, 512), (4, 256), (4, 1024), (8, 256)])
def test_fused_b1_matches_oracle(K, f):
    cfg = W.scaled(W.DECODE35, E=24, K=K, f=f, L=3, B=1)
    L = cfg.L
    _, st, slot_of = _setup(cfg, L)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, K)
    ws = U.empty((E().workspace_bytes(E().E0_OP_STAGED_DECODE, dims, L, 1, 0),), "uint8")
    err = U.zeros((1,), "int32")
    y = U.empty((L, 1, cfg.d))
    x = np.stack([W.activations(cfg, 0, l) for l in range(L)])
    idx, w = _routing(cfg, L, 0)
    E().e0_moe_staged_decode(dims, L, 1, U.f16(x), U.i32(idx), U.f32(w), slot_of, cfg.E, st, None, y, ws, err)
    U.torch().cuda.synchronize()
    assert int(err.item()) == 0
    yh = y.cpu().numpy()
    rs = [U.assert_close(yh[l, 0], _ref_layer(cfg, l, x[l, 0], idx[l, 0], w[l, 0]), TOL, ELEM, l)[0] for l in range(L)]
    print("fused b1", K, f, rs)
    assert max(rs) <= TOL


def test_fused_b1_back_to_back_and_dirty_workspace():
    cfg = W.scaled(W.DECODE35, E=24, L=2, B=1)
    L = cfg.L
    _, st, slot_of = _setup(cfg, L)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    nbytes = E().workspace_bytes(E().E0_OP_STAGED_DECODE, dims, L, 1, 0)
    rng = np.random.default_rng(7)
    ws = U.torch().from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).to(U.dev())
    err = U.zeros((1,), "int32")
    ys, ins = [], []
    for t in range(3):
        x = np.stack([W.activations(cfg, t, l) for l in range(L)])
        idx, w = _routing(cfg, L, t)
        y = U.empty((L, 1, cfg.d))
        E().e0_moe_staged_decode(dims, L, 1, U.f16(x), U.i32(idx), U.f32(w), slot_of, cfg.E, st, None, y, ws, err)
        ys.append(y)
        ins.append((x, idx, w))
    U.torch().cuda.synchronize()
    assert int(err.item()) == 0
    for t in range(3):
        x, idx, w = ins[t]
        yh = ys[t].cpu().numpy()
        for l in range(L):
            U.assert_close(yh[l, 0], _ref_layer(cfg, l, x[l, 0], idx[l, 0], w[l, 0]), TOL, ELEM, (t, l))


def test_fused_b1_errors_flag_and_skip():
    cfg = W.scaled(W.DECODE35, E=24, L=2, B=1)
    L = cfg.L
    _, st, _ = _setup(cfg, L)
    so = np.tile(np.arange(cfg.E, dtype=np.int32), (L, 1))
    so[1, 7] = -1  # expert 7 of layer 1 not resident
    slot_of = U.i32(so)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    ws = U.empty((E().workspace_bytes(E().E0_OP_STAGED_DECODE, dims, L, 1, 0),), "uint8")
    x = np.stack([W.activations(cfg, 0, l) for l in range(L)])
    idx = np.array([[[3, 5, 30, 1]], [[7, 2, 9, 11]]], np.int32)  # 30 >= E; 7 not resident
    w = np.array([[[0.4, 0.3, 0.2, 0.1]], [[0.1, 0.2, 0.3, 0.4]]], np.float32)
    err = U.zeros((1,), "int32")
    y = U.empty((L, 1, cfg.d))
    E().e0_moe_staged_decode(dims, L, 1, U.f16(x), U.i32(idx), U.f32(w), slot_of, cfg.E, st, None, y, ws, err)
    U.torch().cuda.synchronize()
    assert int(err.item()) == E().E0_DEV_BAD_ID | E().E0_DEV_NOT_RESIDENT
    yh = y.cpu().numpy()
    for l, skip in ((0, 2), (1, 0)):
        keep = [k for k in range(cfg.K) if k != skip]
        ref = _ref_layer(cfg, l, x[l, 0], idx[l, 0][keep], w[l, 0][keep])
        U.assert_close(yh[l, 0], ref, TOL, ELEM, l)


def test_fused_b1_shared_expert_with_lora():
    cfg = W.scaled(W.PREROUTED35, E=24, L=2)
    L = cfg.L
    _, st, slot_of = _setup(cfg, L)
    from e0inputs import gpu as G
    bb_sh = gen.bundle_bytes(cfg.d, cfg.shared_f)
    sh_store = U.zeros((L, bb_sh), "uint8")
    for l in range(L):
        G.fill_experts(sh_store[l].data_ptr(), bb_sh, cfg.seed, l, [0], cfg.d, cfg.shared_f, tag=gen.TAG_SHARED)
    lor = [W.lora(cfg, l) for l in range(L)]
    la = [U.f16(np.stack([lor[l][p][0] for l in range(L)])) for p in range(3)]
    lb = [U.f16(np.stack([lor[l][p][1] for l in range(L)])) for p in range(3)]
    shared = E().shared_from_tensors(sh_store, cfg.d, cfg.shared_f, la, lb, cfg.lora_alpha_over_r)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, cfg.K)
    ws = U.empty((E().workspace_bytes(E().E0_OP_STAGED_DECODE, dims, L, 1, cfg.lora_r),), "uint8")
    err = U.zeros((1,), "int32")
    y = U.empty((L, 1, cfg.d))
    x = np.stack([W.activations(cfg, 0, l) for l in range(L)])
    idx, w = _routing(cfg, L, 0)
    E().e0_moe_staged_decode(dims, L, 1, U.f16(x), U.i32(idx), U.f32(w), slot_of, cfg.E, st, shared, y, ws, err)
    U.torch().cuda.synchronize()
    assert int(err.item()) == 0
    yh = y.cpu().numpy()
    for l in range(L):
        sh = oracle.shared_lora(W.shared_expert(cfg, l), lor[l], cfg.lora_r, cfg.lora_alpha_over_r, x[l, 0], cfg.d,
                                cfg.shared_f)
        ref = _ref_layer(cfg, l, x[l, 0], idx[l, 0], w[l, 0]) + sh
        U.assert_close(yh[l, 0], ref, TOL, ELEM, l)
