"""GPU parity of the staged decode at the edges of its routing width: one
expert per token (K = 1, the single-launch kernel), K = 16 and K = 32 = E
(above the single-launch kernel's K <= 8: the two-launch kernels at B = 1,
the sorted batched kernels at B = 2), every expert resident (slot = expert
id). Every token against the fp64 oracle (rel-L2 <= 1e-3 and per token max
|y - ref| <= 1e-4 max |ref|)."""
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


@pytest.mark.parametrize("K,B", [(1, 1), (16, 1), (32, 1), (32, 2), (1, 9)])
def test_staged_decode_routing_width(K, B):
    cfg = W.scaled(W.DECODE8_B32, L=1, B=B, K=K, E=32)
    d, f, Ex = cfg.d, cfg.f, cfg.E
    bb = gen.bundle_bytes(d, f)
    pool = U.gpu_store(cfg, [0])
    so = np.arange(Ex, dtype=np.int32)
    x = W.activations(cfg, 4, 0)
    idx, w = oracle.softmax_topk(W.given_logits(cfg, 4, 0).astype(np.float32), K)
    idx = idx.astype(np.int32)
    w = w.astype(np.float32)
    dims = E().moe_dims(d, f, Ex, K)
    ws = U.empty((E().workspace_bytes(E().E0_OP_STAGED_DECODE, dims, 1, B, 0),), "uint8")
    y = U.empty((1, B, d))
    err = U.zeros((1,), "int32")
    E().e0_moe_staged_decode(dims, 1, B, U.f16(x[None]), U.i32(idx[None]), U.f32(w[None]), U.i32(so[None]), Ex,
                             E().stack_from_bundles(pool, d, f, bb, Ex * bb), None, y, ws, err)
    U.torch().cuda.synchronize()
    assert int(err.item()) == 0
    mats = [gen.expert(cfg.seed, 0, e, d, f) for e in range(Ex)]
    ref, _ = oracle.moe_exact(oracle.Experts(mats), d, f, x, idx, w.astype(np.float64))
    got = y.cpu().numpy()[0]
    for t in range(B):
        r, e = U.assert_close(got[t], ref[t], TOL, ELEM, (K, B, t))
    print(f"K={K} B={B}: last token rel-L2 {r:.3g}, largest element error / max {e:.3g}")
