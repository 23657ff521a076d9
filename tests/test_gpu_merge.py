"""GPU parity: e0_lora_merge_requant (a LoRA delta merged into an int4 g64
matrix and requantised) against the oracle (oracle/merge.py), bit-exact on
codes, scales and biases: the merged codes are decided from fp32 values with
every operation rounded on its own on both sides. Covers the pages' delta
magnitude (RMS about 1e-3) and a large one, ragged shapes (one tile, a
partial block of groups), rank 1 and 64, a zero delta, constant groups, and
an expert's gate and down matrices at full size."""
import numpy as np
import pytest

from e0inputs import gen
from oracle import merge as M
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def E():
    from int4_gather_swiglu_amd import _lib
    return _lib


def _inputs(rows, cols, r, std, seed=21):
    q, s, b = gen.quant_matrix(gen.stream_key(seed, rows, cols, 1), gen.stream_key(seed, rows, cols, 2),
                               gen.stream_key(seed, rows, cols, 3), rows, cols)
    lb = gen.normal_f16(gen.stream_key(seed, rows, cols, 4), rows * r, std).view(np.uint16).reshape(rows, r)
    la = gen.normal_f16(gen.stream_key(seed, rows, cols, 5), r * cols, std).view(np.uint16).reshape(r, cols)
    return q, s, b, lb, la


def _gpu(q, s, b, lb, la, alpha):
    T = U.torch()
    rows, cols = q.shape[0], q.shape[1] * 8
    r = lb.shape[1]
    ngrp = cols // 64
    d = U.dev()
    t = lambda a, dt: T.from_numpy(np.ascontiguousarray(a).view(dt)).to(d)
    qd = t(q, np.int32)
    sd = t(gen._tile8(s).reshape(-1), np.int16)
    bd = t(gen._tile8(b).reshape(-1), np.int16)
    lbd, lad = t(lb, np.int16), t(la, np.int16)
    qo = T.empty_like(qd)
    so = T.empty((rows * ngrp,), dtype=T.int16, device=d)
    bo = T.empty_like(so)
    E().e0_lora_merge_requant(rows, cols, qd, sd, bd, lbd, lad, r, alpha, qo, so, bo)
    T.cuda.synchronize()
    return (qo.cpu().numpy().view(np.uint32),
            gen._untile8(so.cpu().numpy().view(np.uint16), rows, ngrp),
            gen._untile8(bo.cpu().numpy().view(np.uint16), rows, ngrp))


def _check(q, s, b, lb, la, alpha=2.0):
    got = _gpu(q, s, b, lb, la, alpha)
    ref = M.merge_requant(q, s, b, lb, la, alpha)
    for g, e, name in zip(got, ref, ("codes", "scales", "biases")):
        bad = int(np.count_nonzero(g != e))
        assert bad == 0, f"{name}: {bad} of {g.size} differ"
    return got


@pytest.mark.parametrize("rows,cols,r,std", [(64, 512, 16, 0.0112), (64, 512, 16, 0.112), (8, 64, 1, 0.05),
                                             (16, 64 * 40, 64, 0.01), (24, 192, 5, 0.3)])
def test_merge_matches_oracle(rows, cols, r, std):
    _check(*_inputs(rows, cols, r, std))


def test_zero_delta_and_constant_groups():
    q, s, b, lb, la = _inputs(32, 256, 8, 0.05)
    _check(q, s, b, np.zeros_like(lb), np.zeros_like(la))
    s0 = s.copy()
    s0[:, ::2] = 0  # every other group constant (scale 0): merged scale 0 where the delta is zero too
    got = _check(q, s0, b, np.zeros_like(lb), np.zeros_like(la))
    assert np.all(got[1][:, ::2] == 0)


@pytest.mark.parametrize("rows,cols", [(512, 2048), (2048, 512)])
def test_merge_full_expert_matrix(rows, cols):
    q, s, b, lb, la = _inputs(rows, cols, 16, 0.0112)
    got = _check(q, s, b, lb, la)
    ret = M.retention((q, s, b), got, lb, la, 2.0)
    print(f"{rows}x{cols} r=16 delta RMS ~1e-3: retention {ret:.3f}")
