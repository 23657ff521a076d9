"""GPU parity of the batched (B > 1) staged decode with the shared expert and
its unmerged LoRA, at d_model 2048 with d_ff 256, 512 and 1024 (the matrix-core
down kernel at 256 and 512, the vector down kernel at 1024), and at d_model
1024 and 4096 (other gate/up lane layouts), and at the largest batch (64), on a workspace
filled with 0xFF bytes before the call (no stale h row may reach an output).
Every token of every layer against the fp64 oracle: the routed experts'
staged sum plus the shared expert with its LoRA terms."""
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


@pytest.mark.parametrize("d,f,B", [(2048, 256, 5), (2048, 512, 5), (2048, 1024, 5), (1024, 128, 5), (4096, 512, 5),
                                   (2048, 512, 64)])
def test_batched_decode_shared_expert_with_lora(d, f, B):
    cfg = W.scaled(W.PREROUTED35, E=24, L=2, B=B, d=d, f=f, shared_f=f)
    L, B, K, d = cfg.L, cfg.B, cfg.K, cfg.d
    from e0inputs import gpu as G
    store = U.gpu_store(cfg, range(L))
    bb = gen.bundle_bytes(d, f)
    st = E().stack_from_bundles(store, d, f, bb, cfg.E * bb)
    slot_of = U.i32(np.tile(np.arange(cfg.E, dtype=np.int32), (L, 1)))
    sh_store = U.zeros((L, bb), "uint8")
    for l in range(L):
        G.fill_experts(sh_store[l].data_ptr(), bb, cfg.seed, l, [0], d, f, tag=gen.TAG_SHARED)
    lor = [W.lora(cfg, l) for l in range(L)]
    la = [U.f16(np.stack([lor[l][p][0] for l in range(L)])) for p in range(3)]
    lb = [U.f16(np.stack([lor[l][p][1] for l in range(L)])) for p in range(3)]
    shared = E().shared_from_tensors(sh_store, d, f, la, lb, cfg.lora_alpha_over_r)
    dims = E().moe_dims(d, f, cfg.E, K)
    ws = U.empty((E().workspace_bytes(E().E0_OP_STAGED_DECODE, dims, L, B, cfg.lora_r),), "uint8")
    ws.fill_(0xFF)
    err = U.zeros((1,), "int32")
    y = U.empty((L, B, d))
    x = np.stack([W.activations(cfg, 0, l) for l in range(L)])
    idx = np.zeros((L, B, K), np.int32)
    w = np.zeros((L, B, K), np.float32)
    for l in range(L):
        i, ww = oracle.softmax_topk(W.given_logits(cfg, 0, l).astype(np.float32), K)
        idx[l], w[l] = i, ww
    E().e0_moe_staged_decode(dims, L, B, U.f16(x), U.i32(idx), U.f32(w), slot_of, cfg.E, st, shared, y, ws, err)
    U.torch().cuda.synchronize()
    assert int(err.item()) == 0
    yh = y.cpu().numpy()
    for l in range(L):
        ids = sorted(set(int(e) for e in idx[l].ravel()))
        mats = {e: gen.expert(cfg.seed, l, e, d, f) for e in ids}
        lst = [mats.get(e, mats[ids[0]]) for e in range(cfg.E)]
        ref, _ = oracle.moe_exact(oracle.Experts(lst), d, f, x[l], idx[l], w[l].astype(np.float64))
        shx = W.shared_expert(cfg, l)
        for t in range(B):
            sh = oracle.shared_lora(shx, lor[l], cfg.lora_r, cfg.lora_alpha_over_r, x[l, t], d, f)
            U.assert_close(yh[l, t], ref[t] + sh, TOL, ELEM, (l, t))
