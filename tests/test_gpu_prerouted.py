"""GPU parity: the prerouted pipeline at the 35B shape (32 staged layers,
heads over [hidden | current K-hot | previous K-hot] = 2560, fc1 -> erf-GELU
-> fc2 plus the linear residual, prediction used as the routing, slot update
of changed experts, staged decode with the shared expert and its unmerged
rank-16 LoRA). Predicted routing and slot tables bit-exact; outputs rel-L2 <=
1e-3; the heads' logits element by element within LOGIT_ATOL of the oracle's
fp64 logits. Planted hiddens are redrawn until every routing decision of the
oracle's head logits has a margin >= 1e-3.

LOGIT_ATOL: the kernel accumulates fp16 products in fp32 over 2560 (fc1),
512 (fc2) and 2048 (linear residual) inputs whose absolute sums stay below
about 40 here; a few dozen roundings of 2^-24 relative to that is under 1e-5,
and erf in fp32 adds less. 1e-4 leaves a margin and is about a thousandth of
what the fc1 -> GELU -> fc2 branch contributes to a logit (about 0.2), so an
error in that branch, which the planted +8 .. +6.5 targets hide from the
routing ids, still fails."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-3
DELTA = 1e-3
LOGIT_ATOL = 1e-4


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _device_model(cfg, L):
    T = U.torch()
    heads = [W.head(cfg, j) for j in range(L)]
    st = lambda arrs: U.f16(np.stack(arrs))
    dh = dict(fc1_w=st([h.fc1_w for h in heads]), fc1_b=st([h.fc1_b for h in heads]),
              fc2_w=st([h.fc2_w for h in heads]), fc2_b=st([h.fc2_b for h in heads]),
              lin_w=st([h.lin_w for h in heads]))
    bb_sh = gen.bundle_bytes(cfg.d, cfg.shared_f)
    sh_store = U.zeros((L, bb_sh), "uint8")
    from e0inputs import gpu as G
    for l in range(L):
        G.fill_experts(sh_store[l].data_ptr(), bb_sh, cfg.seed, l, [0], cfg.d, cfg.shared_f, tag=gen.TAG_SHARED)
    lor = [W.lora(cfg, l) for l in range(L)]
    la = [U.f16(np.stack([lor[l][p][0] for l in range(L)])) for p in range(3)]
    lb = [U.f16(np.stack([lor[l][p][1] for l in range(L)])) for p in range(3)]
    del T
    return heads, dh, sh_store, la, lb, lor


def test_prerouted35b_pipeline_steps():
    cfg = W.PREROUTED35
    L, K, steps = cfg.L, cfg.K, 4
    heads, dh, sh_store, la, lb, lor = _device_model(cfg, L)
    # Oracle routing state while drawing the inputs (tie-free heads).
    P0 = W.prerouted_inputs  # noqa: F841
    owner0 = np.empty((steps, K), np.int32)
    owner0[0] = W.initial_set(cfg, -1)
    for t in range(1, steps):
        owner0[t] = W.next_set(cfg, owner0[t - 1], t, -1)
    R = {0: np.concatenate([owner0[0][None], np.stack([W.initial_set(cfg, l) for l in range(L)])])}
    Wt = {}
    for t in range(1, steps + 1):
        R[t] = np.zeros((L + 1, K), np.int32)
        Wt[t] = np.zeros((L + 1, K), np.float64)
        if t < steps:
            R[t][0] = owner0[t]

    O = {}

    def accept(t, j, h):
        cur = R[t][j]
        prev = R[t - 1][j] if t > 0 else None
        o64 = oracle.head_logits(heads[j], h, cur, prev, K)
        o = o64.astype(np.float32)[None]
        if oracle.route_margin(o, cfg) < DELTA:
            return False
        O[(t, j)] = o64
        idx, w = oracle.softmax_topk(o, K)
        R[t + 1][j + 1] = idx[0]
        Wt[t + 1][j + 1] = w[0]
        return True

    P = W.prerouted_inputs(cfg, steps, accept=accept)
    # Device pipeline.
    from int4_gather_swiglu_amd.pipeline import PrerouterPipeline
    Tt = U.torch()
    store = U.gpu_store(cfg, range(L))
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    pool = U.zeros((L, cfg.S, bb), "uint8")
    st_store = E().stack_from_bundles(store, cfg.d, cfg.f, bb, cfg.E * bb)
    st_pool = E().stack_from_bundles(pool, cfg.d, cfg.f, bb, cfg.S * bb)
    shared = E().shared_from_tensors(sh_store, cfg.d, cfg.shared_f, la, lb, cfg.lora_alpha_over_r)
    hd = E().heads_from_tensors(dh["fc1_w"], dh["fc1_b"], dh["fc2_w"], dh["fc2_b"], dh["lin_w"])
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, K)
    pipe = PrerouterPipeline(dims, L, 1, cfg.S, st_store, st_pool, hd, E().route_params(0, K), shared=shared)
    Rd = U.zeros((steps + 1, L + 1, 1, K), "int32")
    Wd = U.zeros((steps + 1, L + 1, 1, K))
    Rd[0, :, 0] = U.i32(R[0])
    Wd[0, 1:, 0] = 1.0 / K
    for t in range(1, steps):
        Rd[t, 0, 0] = U.i32(owner0[t])
    hin = U.f16(P.hin[:, :, None, :])  # [steps][L+1][1][d]
    ys = U.empty((steps, L, 1, cfg.d))
    lo = U.empty((steps, L, 1, cfg.E))
    recs = []
    pipe.update_ids(Rd[0, 1:], None)
    pipe.join()
    for t in range(steps):
        pipe.predict(hin[t], Rd[t], Rd[t - 1] if t > 0 else None, Rd[t + 1], Wd[t + 1], logits_out=lo[t])
        Tt.cuda.current_stream().synchronize()
        pipe.side.synchronize()
        recs.append(dict(slot_of=pipe.slot_of.cpu().numpy(), expert_of=pipe.expert_of.cpu().numpy()))
        pipe.update_ids(Rd[t + 1, 1:], Rd[t, 1:])
        pipe.decode_ids(Rd[t, 1:], Wd[t, 1:], hin[t, 1:], ys[t])
        pipe.join()
    Tt.cuda.synchronize()
    assert int(pipe.err.item()) == 0
    Rh = Rd.cpu().numpy()[:, :, 0]
    Wh = Wd.cpu().numpy()[:, :, 0]
    # 1. predicted routing bit-exact, weights close
    for t in range(1, steps + 1):
        assert np.array_equal(Rh[t, 1:], R[t][1:]), t
        assert np.abs(Wh[t, 1:] - Wt[t][1:]).max() < 1e-5
    rep = np.mean([len(set(Rh[t, 1 + l]) & set(Rh[t - 1, 1 + l])) / K for t in range(2, steps + 1) for l in range(L)])
    print("realized repeat rate", rep)
    # 1b. every head's logits, element by element
    lh = lo.cpu().numpy()[:, :, 0]
    dl = max(float(np.abs(lh[t, j] - O[(t, j)]).max()) for t in range(steps) for j in range(L))
    print("head logits: largest |gpu - oracle|", dl)
    assert dl <= LOGIT_ATOL
    # 2. slot tables bit-exact against the oracle's rule
    so = np.full((L, cfg.E), -1, np.int32)
    eo = np.full((L, cfg.S), -1, np.int32)
    for t in range(steps):
        for l in range(L):
            rc, _ = oracle.slot_update(cfg.E, cfg.S, Rh[t, 1 + l], Rh[t - 1, 1 + l] if t > 0 else [], so[l], eo[l])
            assert rc == 0
        assert np.array_equal(recs[t]["slot_of"], so) and np.array_equal(recs[t]["expert_of"], eo), t
    # 3. outputs: routed + shared expert with LoRA, sampled layers
    y = ys.cpu().numpy()
    rs = []
    for t, l in [(0, 0), (1, 13), (2, 31), (3, 7)]:
        x = P.hin[t, 1 + l][None]
        ids = Rh[t, 1 + l]
        mats = {int(e): gen.expert(cfg.seed, l, int(e), cfg.d, cfg.f) for e in ids}
        lst = [mats.get(e, mats[int(ids[0])]) for e in range(cfg.E)]
        routed, _ = oracle.moe_exact(oracle.Experts(lst), cfg.d, cfg.f, x, ids[None], Wh[t, 1 + l][None].astype(np.float64))
        sh = oracle.shared_lora(W.shared_expert(cfg, l), lor[l], cfg.lora_r, cfg.lora_alpha_over_r, x[0], cfg.d, cfg.shared_f)
        ref = routed[0] + sh
        rs.append(U.assert_close(y[t, l, 0], ref, TOL, 1e-4, (t, l))[0])
    print("prerouted rel-L2", rs)
    assert max(rs) <= TOL
