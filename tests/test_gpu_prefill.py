"""GPU parity: sorted whole-layer prefill (sort by expert, MFMA grouped GEMM,
weighted combine) against the fp64 oracle, rel-L2 <= 1e-3 and, per token,
max |y - ref| <= ELEM * max |ref|. fp16 MFMA operands (x exact; weights and
the SwiGLU hidden rounded to fp16, each within 2^-11 relative; experts of
at most 16 rows take the codes as exact fp16 denormals with scale and bias
applied in fp32, so only the hidden is rounded there) put the expected
rel-L2 near 4e-4; the largest element error of a row is then about
as large relative to the row's largest value, and ELEM = 3e-3 leaves a
margin while a wrong 32-row block or column block (an O(1) error on a few
elements) still fails."""
import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-3
ELEM = 3e-3


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _prefill(cfg, store_layer, x, idx, w):
    """Run e0_moe_sorted_prefill on device tensors; returns y (host) and err."""
    T = x.shape[0]
    bb = gen.bundle_bytes(cfg.d, cfg.f)
    dims = E().moe_dims(cfg.d, cfg.f, cfg.E, idx.shape[1])
    st = E().stack_from_bundles(store_layer, cfg.d, cfg.f, bb, 0)
    ws = U.empty((E().workspace_bytes(E().E0_OP_SORTED_PREFILL, dims, T),), "uint8")
    y = U.empty((T, cfg.d))
    err = U.zeros((1,), "int32")
    E().e0_moe_sorted_prefill(dims, T, U.f16(x), U.i32(idx), U.f32(w), st, y, ws, err)
    U.torch().cuda.synchronize()
    return y.cpu().numpy(), int(err.item())


def _oracle(cfg, layer, x, idx, w, tokens):
    ids = sorted(set(idx[tokens].ravel().tolist()) - {-1})
    mats = {e: gen.expert(cfg.seed, layer, e, cfg.d, cfg.f) for e in ids if 0 <= e < cfg.E}
    first = next(iter(mats.values()))
    lst = [mats.get(e, first) for e in range(cfg.E)]
    idx_s = idx[tokens].copy()
    w_s = w[tokens].astype(np.float64)
    bad = (idx_s < 0) | (idx_s >= cfg.E)
    idx_s[bad] = ids[0]
    w_s[bad] = 0.0
    ref, _ = oracle.moe_exact(oracle.Experts(lst), cfg.d, cfg.f, x[tokens], idx_s, w_s)
    return ref


def test_tiny_prefill_all_tokens():
    cfg = W.scaled(W.TINY, B=37)
    store = U.gpu_store(cfg, [0])[0]
    x = W.activations(cfg, 0, 0)
    lg = W.given_logits(cfg, 0, 0).astype(np.float32)
    idx, w = oracle.softmax_topk(lg, cfg.K)
    y, err = _prefill(cfg, store, x, idx, w.astype(np.float32))
    assert err == 0
    ref = _oracle(cfg, 0, x, idx, w.astype(np.float32), np.arange(cfg.B))
    print("tiny prefill rel-L2, elem", U.assert_close(y, ref, TOL, ELEM))


@pytest.mark.parametrize("T", [1, 5, 128, 300])
def test_tiny_prefill_ragged_and_single_token(T):
    cfg = W.scaled(W.TINY, B=T)
    store = U.gpu_store(cfg, [0])[0]
    x = W.activations(cfg, 1, 0)
    idx, w = oracle.softmax_topk(W.given_logits(cfg, 1, 0).astype(np.float32), cfg.K)
    y, err = _prefill(cfg, store, x, idx, w.astype(np.float32))
    assert err == 0
    tok = np.unique(np.linspace(0, T - 1, min(T, 24)).astype(int))
    U.assert_close(y[tok], _oracle(cfg, 0, x, idx, w.astype(np.float32), tok), TOL, ELEM)


def test_prefill_one_expert_takes_every_token():
    cfg = W.scaled(W.TINY, B=300)
    store = U.gpu_store(cfg, [0])[0]
    x = W.activations(cfg, 2, 0)
    idx = np.tile(np.array([[5, 2, 9, 0]], np.int32), (cfg.B, 1))
    idx[::3, 1] = 7  # a second popular expert on a third of the tokens
    w = np.tile(np.array([[0.4, 0.3, 0.2, 0.1]], np.float32), (cfg.B, 1))
    y, err = _prefill(cfg, store, x, idx, w)
    assert err == 0
    tok = np.arange(0, cfg.B, 13)
    U.assert_close(y[tok], _oracle(cfg, 0, x, idx, w, tok), TOL, ELEM)


@pytest.mark.parametrize("d,f", [(4096, 256), (2176, 384)])
def test_prefill_tails_at_the_small_tile_bound(d, f):
    # Expert row counts chosen around the 16-row bound of the matrix-core
    # path for small experts: 1 and 16 on it; 2 (the tail of 130: a tail of a
    # larger expert stays on the 32-row blocks), 17, 20, 30, 86 on the 32-row
    # blocks. d = 4096 gives 64 groups (two 32-group bias
    # products); d = 2176 gives 34 (a partial second one) and a d_model that
    # is not a multiple of 256 (down in 128-column blocks); the down
    # reductions (4 and 6 groups) fill part of one bias product. Every token.
    cfg = W.scaled(W.TINY, d=d, f=f, E=8, K=2, B=150)
    store = U.gpu_store(cfg, [0])[0]
    x = W.activations(cfg, 5, 0)
    t = np.arange(cfg.B)
    idx = np.stack([np.where(t < 130, 3, 5),
                    np.select([t < 16, t < 33, t == 33, t < 120], [0, 1, 2, 4], 6)], axis=1).astype(np.int32)
    assert sorted(np.bincount(idx.ravel(), minlength=cfg.E).tolist()) == [0, 1, 16, 17, 20, 30, 86, 130]
    w = (0.1 + 0.9 * gen.uniform24(gen.draws(gen.stream_key(cfg.seed, gen.TAG_LOGITS, 99), cfg.B * cfg.K)))
    w = w.reshape(cfg.B, cfg.K)
    y, err = _prefill(cfg, store, x, idx, w)
    assert err == 0
    r, e = U.assert_close(y, _oracle(cfg, 0, x, idx, w, t), TOL, ELEM, f"small-tile bound d={d} f={f}")
    print(f"small-tile bound d={d} f={f}: rel-L2 {r:.3g}, largest element error / row max {e:.3g}")


@pytest.mark.parametrize("E,K,T", [(1024, 8, 200), (64, 1, 500), (16, 16, 40)])
def test_prefill_routing_width_extremes(E, K, T):
    # The widest expert count the call takes (1024: the sort's counters per
    # thread), one expert per token, and every expert for every token (K = E).
    cfg = W.scaled(W.TINY, E=E, K=K, B=T)
    store = U.gpu_store(cfg, [0])[0]
    x = W.activations(cfg, 6, 0)
    idx, w = oracle.softmax_topk(W.given_logits(cfg, 6, 0).astype(np.float32), K)
    w = w.astype(np.float32)
    y, err = _prefill(cfg, store, x, idx, w)
    assert err == 0
    r, e = U.assert_close(y, _oracle(cfg, 0, x, idx, w, np.arange(T)), TOL, ELEM, f"E={E} K={K} T={T}")
    print(f"E={E} K={K} T={T}: rel-L2 {r:.3g}, largest element error / row max {e:.3g}")


def test_prefill_bad_ids_flag_and_skip():
    cfg = W.scaled(W.TINY, B=16)
    store = U.gpu_store(cfg, [0])[0]
    x = W.activations(cfg, 3, 0)
    idx, w = oracle.softmax_topk(W.given_logits(cfg, 3, 0).astype(np.float32), cfg.K)
    idx[3, 2] = cfg.E
    idx[7, 0] = -1
    w = w.astype(np.float32)
    y, err = _prefill(cfg, store, x, idx, w)
    assert err == E().E0_DEV_BAD_ID
    U.assert_close(y, _oracle(cfg, 0, x, idx, w, np.arange(cfg.B)), TOL, ELEM)


def _by_expert(cfg, x, idx, w):
    """Every token at once: each active expert dequantised once, fp64 products."""
    return oracle.moe_by_expert(lambda e: gen.expert(cfg.seed, 0, e, cfg.d, cfg.f), cfg.E, cfg.d, cfg.f, x, idx, w)


def test_tiny_prefill_13k_pairs_every_token():
    # T*K = 13,200 pairs (the pages' ~3.3k-token prompt at K = 4): more pairs
    # than the sort loads in one batch, so its later batches run; every token
    # compared.
    cfg = W.scaled(W.TINY, B=3300)
    store = U.gpu_store(cfg, [0])[0]
    x = W.activations(cfg, 4, 0)
    idx, w = oracle.softmax_topk(W.given_logits(cfg, 4, 0).astype(np.float32), cfg.K)
    w = w.astype(np.float32)
    y, err = _prefill(cfg, store, x, idx, w)
    assert err == 0
    print("tiny T=3300 rel-L2, elem", U.assert_close(y, _by_expert(cfg, x, idx, w), TOL, ELEM))


def _routed_on_gpu(cfg, lg16):
    """Routing on the GPU (as the bench does), checked bit-exact against the oracle."""
    T = cfg.B
    p = E().route_params(0, cfg.K)
    idx_d = U.empty((1, T, cfg.K), "int32")
    w_d = U.empty((1, T, cfg.K))
    E().e0_route(p, 1, T, cfg.E, U.f16(lg16[None]), True, None, None, 0, idx_d, w_d, None)
    U.torch().cuda.synchronize()
    idx = idx_d.cpu().numpy()[0]
    w = w_d.cpu().numpy()[0]
    ridx, _ = oracle.softmax_topk(lg16.astype(np.float32), cfg.K)
    assert np.array_equal(idx, ridx)
    return idx, w


@pytest.mark.parametrize("T", [2048, 3300])
def test_prefill35b_zipf_full_shape_every_token(T):
    # The 35B-tier layer with Zipf(1.1) popularity at the workload's T = 2048
    # and at the pages' prompt length (13,200 pairs): every token compared, so
    # every M-tile of every active expert (heavy, mid and tail classes) and
    # every column block is checked.
    cfg = W.scaled(W.PREFILL35, B=T)
    store = U.gpu_store(cfg, [0])[0]
    x = W.activations(cfg, 0, 0)
    idx, w = _routed_on_gpu(cfg, W.given_logits(cfg, 0, 0))
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    print("active experts", int((counts > 0).sum()), "top count", int(counts.max()),
          "experts < 16 rows", int(((counts > 0) & (counts < 16)).sum()))
    y, err = _prefill(cfg, store, x, idx, w)
    assert err == 0
    r, e = U.assert_close(y, _by_expert(cfg, x, idx, w), TOL, ELEM, f"prefill35b T={T}")
    print(f"prefill35b T={T}: rel-L2 {r:.3g}, largest element error / row max {e:.3g}")
