"""GPU parity of e0_prerouter away from the prerouted tier's own shape: a
d_model above 2048 (the general fc1 kernel: one wavefront per row, the hidden
part streamed), several tokens per head, E = 128 with K = 8, no previous
token (prev_idx NULL: only the current K-hot columns), and the sigmoid-group
rule (the 8B tier's routing) on the predicted logits. The logits are compared
element by element with the oracle's fp64 head; the routed ids wherever the
oracle's selection margin on its logits exceeds what the logits' error can
move, the weights within 1e-5."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
LOGIT_ATOL = 1e-4
MARGIN = 1e-3


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


@pytest.mark.parametrize("d,Ex,K,B,with_prev,mode", [(4096, 128, 8, 3, True, 0), (2048, 256, 4, 5, False, 0),
                                                      (8192, 64, 2, 2, True, 0), (2048, 128, 8, 4, True, 1)])
def test_prerouter_shapes(d, Ex, K, B, with_prev, mode):
    grp = dict(mode=1, n_groups=8, topk_groups=4, scale=2.5) if mode else {}
    cfg = W.scaled(W.PREROUTED35, d=d, E=Ex, K=K, L=3, **grp)
    H = cfg.L
    heads = [W.head(cfg, j) for j in range(H)]
    st = lambda arrs: U.f16(np.stack(arrs))
    hd = E().heads_from_tensors(st([h.fc1_w for h in heads]), st([h.fc1_b for h in heads]),
                                st([h.fc2_w for h in heads]), st([h.fc2_b for h in heads]),
                                st([h.lin_w for h in heads]))
    rng = np.random.default_rng(d + Ex)
    h = gen.normal_f16(gen.stream_key(cfg.seed, gen.TAG_ACT, 91, d), H * B * d).reshape(H, B, d)
    cur = np.stack([[rng.choice(Ex, size=K, replace=False) for _ in range(B)] for _ in range(H)]).astype(np.int32)
    prev = np.stack([[rng.choice(Ex, size=K, replace=False) for _ in range(B)] for _ in range(H)]).astype(np.int32)
    dims = E().moe_dims(d, heads[0].fc1_w.shape[0], Ex, K)
    ws = U.empty((E().workspace_bytes(E().E0_OP_PREROUTER, dims, H, B, 0),), "uint8")
    idx, w, lo = U.empty((H, B, K), "int32"), U.empty((H, B, K)), U.empty((H, B, Ex))
    E().e0_prerouter(hd, H, B, d, Ex, U.f16(h), U.i32(cur), U.i32(prev) if with_prev else None,
                     E().route_params(cfg.mode, K, cfg.n_groups, cfg.topk_groups, cfg.scale), idx, w, lo, ws)
    U.torch().cuda.synchronize()
    gi, gw, gl = idx.cpu().numpy(), w.cpu().numpy(), lo.cpu().numpy()
    worst, checked = 0.0, 0
    for j in range(H):
        for b in range(B):
            ref = oracle.head_logits(heads[j], h[j, b], cur[j, b], prev[j, b] if with_prev else None, K)
            worst = max(worst, float(np.abs(gl[j, b] - ref).max()))
            r32 = ref.astype(np.float32)[None]
            if oracle.route_margin(r32, cfg) > MARGIN:
                ri, rw = oracle.route(r32, cfg)
                assert np.array_equal(gi[j, b], ri[0]), (j, b)
                assert np.abs(gw[j, b] - rw[0]).max() < 1e-5, (j, b)
                checked += 1
    print(f"d={d} E={Ex} K={K} B={B} mode={mode}: largest |logit - oracle| {worst:.3g}, ids checked on {checked}/{H * B} rows")
    assert worst <= LOGIT_ATOL
    assert checked >= H * B // 2
