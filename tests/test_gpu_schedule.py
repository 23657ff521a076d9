"""GPU parity of the schedules the benchmark times, at the full 35B shapes.

The benchmark's own step objects (bench.DecodeSchedule, bench.PrerouterSchedule)
run eight steps: routing or the prerouter heads and the slot update on the side
stream, overlapped with the staged decode of the step on the main stream (the
one-token lead: koala.ai.kr walkthrough, prerouter section and the Fig. 1
timeline; jaehun.me review, appendix B on rewriting slots in place). Checked
against the oracle: routing ids, predicted ids and both slot tables after every
step bit-exact, routing weights within 1e-5, every layer's output within
rel-L2 1e-3 and a per-element bound.

The delayed variants hold the main stream in a bounded spin kernel before each
decode, so the side stream's slot update for step t + 1 has finished before
the decode of step t starts: an update that rewrote a slot step t reads would
show in that step's output. They also compare, on the main stream just before
and just after each decode, the pool bytes of every slot step t reads with the
store's bytes of the expert it should hold (the check after a decode is
enqueued before the side stream may start the next update)."""
import argparse
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from e0inputs import gen, workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-3
ELEM = 1e-4
DELTA = 1e-3
DELAY_CYCLES = 1_000_000  # spin kernel before each decode (well under a millisecond)
STEPS = 8


def _args(steps):
    return argparse.Namespace(steps=steps, warmup=0, host_store=False, hot_slots=0, no_overlap=False)


def _resident_ok(pipe, store, pool, idx):
    """0-dim device bool, enqueued on the current stream: every expert of idx
    [L][B][K] has a slot whose pool bytes equal the store's bytes of it."""
    T = U.torch()
    L = idx.shape[0]
    ids = idx.reshape(L, -1).long()
    slots = pipe.slot_of.gather(1, ids.clamp(0, pipe.slot_of.shape[1] - 1)).long()
    ar = T.arange(L, device=ids.device)[:, None]
    same = (pool[ar, slots.clamp(min=0)] == store[ar, ids]).all()
    return same & (slots >= 0).all()


def _hazard_hook(T, delay, state, checks):
    def pre(t):
        if delay:
            T.cuda._sleep(delay)
        s = state["sch"]
        checks.append(_resident_ok(s.pipe, s.store, s.pool, state["idx"](t)))
    return pre


def _tables_hook(T, pipe_of, tabs):
    """Slot tables right after the update for step t + 1, copied on the stream
    the update ran on (the update for t + 2 may start before main has waited
    for this one)."""
    def hook(t, stream):
        pipe = pipe_of()
        with T.cuda.stream(stream):
            tabs.append((pipe.slot_of.clone(), pipe.expert_of.clone()))
    return hook


def _post_hook(state, post):
    """Right after the decode of step t on main (before the next update may
    start): the slots step t read still hold its experts' bytes."""
    def hook(t):
        s = state["sch"]
        post.append(_resident_ok(s.pipe, s.store, s.pool, state["idx"](t)))
    return hook


def _replay(E, S, routes, L):
    """Oracle slot rule over routes[s] ([L][K] per step); tables after each update."""
    so = np.full((L, E), -1, np.int32)
    eo = np.full((L, S), -1, np.int32)
    out = []
    for s, r in enumerate(routes):
        for l in range(L):
            rc, _ = oracle.slot_update(E, S, r[l], routes[s - 1][l] if s else [], so[l], eo[l])
            assert rc == 0
        out.append((so.copy(), eo.copy()))
    return out


def _ref_layers(cfg, x, idx, w, extra=None):
    """Oracle output of every layer of one step: [L][d]. x [L][d], idx/w [L][K]."""
    def one(l):
        ids = [int(e) for e in idx[l]]
        mats = {e: gen.expert(cfg.seed, l, e, cfg.d, cfg.f) for e in ids}
        lst = [mats.get(e, mats[ids[0]]) for e in range(cfg.E)]
        y, err = oracle.moe_exact(oracle.Experts(lst), cfg.d, cfg.f, x[l][None], idx[l][None],
                                  np.asarray(w[l], np.float64)[None])
        assert err == 0
        return y[0] + (extra(l, x[l]) if extra is not None else 0.0)
    with ThreadPoolExecutor(16) as ex:
        return np.stack(list(ex.map(one, range(idx.shape[0]))))


@pytest.mark.parametrize("delay", [0, DELAY_CYCLES], ids=["overlapped", "main-delayed"])
def test_decode35b_bench_schedule(delay):
    import bench
    T = U.torch()
    cfg = W.DECODE35
    L, K = cfg.L, cfg.K
    checks, state, post, tabs = [], {}, [], []
    sch = bench.DecodeSchedule(_args(STEPS), cfg, STEPS, pre_decode=_hazard_hook(T, delay, state, checks),
                               post_decode=_post_hook(state, post),
                               post_update=_tables_hook(T, lambda: state["sch"].pipe, tabs))
    state["sch"] = sch
    state["idx"] = lambda t: sch.pipe.idx[t % 2]
    pipe = sch.pipe
    rec = [dict(idx=pipe.idx[0].clone(), w=pipe.w[0].clone())]
    ys = []
    for t in range(STEPS):
        sch.step(t, None)
        ys.append(sch.y.clone())
        rec.append(dict(idx=pipe.idx[(t + 1) % 2].clone(), w=pipe.w[(t + 1) % 2].clone()))
    T.cuda.synchronize()
    assert int(pipe.err.item()) == 0
    assert all(bool(c.item()) for c in checks), "a slot read by a step held other bytes before its decode"
    assert all(bool(c.item()) for c in post), "a slot read by a step held other bytes after its decode"
    # routing of steps 0 .. STEPS (the inputs repeat with period STEPS)
    routes = []
    for s in range(STEPS + 1):
        lg = np.stack([W.given_logits(cfg, s % STEPS, l) for l in range(L)]).reshape(L, cfg.E).astype(np.float32)
        ridx, rw = oracle.softmax_topk(lg, K)
        got_i = rec[s]["idx"].cpu().numpy().reshape(L, K)
        assert np.array_equal(got_i, ridx), s
        assert np.abs(rec[s]["w"].cpu().numpy().reshape(L, K) - rw).max() < 1e-5
        routes.append(ridx)
    tables = _replay(cfg.E, sch.S, routes, L)
    worst = (0.0, 0.0)
    for t in range(STEPS):
        so, eo = tables[t + 1]
        assert np.array_equal(tabs[t][0].cpu().numpy(), so), t
        assert np.array_equal(tabs[t][1].cpu().numpy(), eo), t
        x = np.stack([W.activations(cfg, t, l)[0] for l in range(L)])
        ref = _ref_layers(cfg, x, routes[t], rec[t]["w"].cpu().numpy().reshape(L, K))
        r, e = U.assert_close(ys[t].cpu().numpy().reshape(L, cfg.d), ref, TOL, ELEM, f"step {t}")
        worst = (max(worst[0], r), max(worst[1], e))
    print(f"decode35b schedule ({'delayed' if delay else 'overlapped'}): worst rel-L2 {worst[0]:.3g}, "
          f"element {worst[1]:.3g}")
    state.clear()  # the hook refers to the schedule: drop the cycle so its buffers free now


@pytest.mark.parametrize("delay", [0, DELAY_CYCLES], ids=["overlapped", "main-delayed"])
def test_prerouted35b_bench_schedule(delay):
    import bench
    T = U.torch()
    cfg = W.PREROUTED35
    L, K = cfg.L, cfg.K
    P = W.prerouted_inputs(cfg, STEPS)
    heads = [W.head(cfg, j) for j in range(L)]
    lor = [W.lora(cfg, l) for l in range(L)]
    checks, state, post, tabs = [], {}, [], []
    sch = bench.PrerouterSchedule(_args(STEPS), cfg, STEPS, pre_decode=_hazard_hook(T, delay, state, checks),
                                  inputs=P, post_decode=_post_hook(state, post),
                                  post_update=_tables_hook(T, lambda: state["sch"].pipe, tabs))
    state["sch"] = sch
    state["idx"] = lambda t: sch.R[sch.r_of(t), 1:]
    pipe = sch.pipe
    preds, ys = [], []
    for t in range(STEPS):
        sch.step(t, None)
        ys.append(sch.y.clone())
        preds.append((sch.R[sch.r_of(t + 1)].clone(), sch.Wt[sch.r_of(t + 1)].clone()))
    T.cuda.synchronize()
    assert int(pipe.err.item()) == 0
    assert all(bool(c.item()) for c in checks) and all(bool(c.item()) for c in post)
    # Oracle: heads step by step from the oracle's own predictions.
    R = {0: np.concatenate([P.owner0[0][None], P.r0])}
    Wr = {0: np.full((L + 1, K), 1.0 / K)}
    for t in range(STEPS):
        R[t + 1] = np.zeros((L + 1, K), np.int32)
        Wr[t + 1] = np.zeros((L + 1, K))
        R[t + 1][0] = P.owner0[(t + 1) % STEPS]

        def head(j, t=t):
            o = oracle.head_logits(heads[j], P.hin[t, j], R[t][j], R[t - 1][j] if t else None, K)
            o32 = o.astype(np.float32)[None]
            return oracle.route_margin(o32, cfg), oracle.softmax_topk(o32, K)
        with ThreadPoolExecutor(16) as ex:
            res = list(ex.map(head, range(L)))
        for j, (margin, (idx, w)) in enumerate(res):
            assert margin >= DELTA, f"input decision margin {margin} at step {t}, head {j}"
            R[t + 1][j + 1] = idx[0]
            Wr[t + 1][j + 1] = w[0]
        got_i = preds[t][0].cpu().numpy()[:, 0]
        assert np.array_equal(got_i[1:], R[t + 1][1:]), t
        assert np.abs(preds[t][1].cpu().numpy()[1:, 0] - Wr[t + 1][1:]).max() < 1e-5
    tables = _replay(cfg.E, sch.S, [R[s][1:] for s in range(STEPS + 1)], L)

    def shared(l, x):
        return oracle.shared_lora(W.shared_expert(cfg, l), lor[l], cfg.lora_r, cfg.lora_alpha_over_r, x, cfg.d,
                                  cfg.shared_f)
    worst = (0.0, 0.0)
    for t in range(STEPS):
        so, eo = tables[t + 1]
        assert np.array_equal(tabs[t][0].cpu().numpy(), so), t
        assert np.array_equal(tabs[t][1].cpu().numpy(), eo), t
        # the decode's own routing weights (checked above against the oracle's)
        w_t = preds[t - 1][1].cpu().numpy()[1:, 0] if t else np.full((L, K), 1.0 / K, np.float32)
        ref = _ref_layers(cfg, P.hin[t, 1:], R[t][1:], w_t, extra=shared)
        r, e = U.assert_close(ys[t].cpu().numpy().reshape(L, cfg.d), ref, TOL, ELEM, f"step {t}")
        worst = (max(worst[0], r), max(worst[1], e))
    print(f"prerouted35b schedule ({'delayed' if delay else 'overlapped'}): worst rel-L2 {worst[0]:.3g}, "
          f"element {worst[1]:.3g}")
    state.clear()
