"""The five synthetic workloads of the routed-expert int4 SwiGLU hot path.

Shapes, value distributions and structure follow the two release tiers the
pages describe (35B: 40 layers x 256 experts, d_model 2048, expert width 512,
softmax-top-4; 8B: 24 layers x 128 experts, sigmoid-group 8 groups / keep 4 /
scale 2.5, top-8; int4 affine group-64 everywhere; prerouter heads over
[hidden | current K-hot | previous K-hot] = 2048 + 2*256 wide, hidden width
512; recovery LoRA r=16, alpha=32). Every value is drawn from ``gen`` streams;
nothing here computes any part of the method.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import gen


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    d: int
    f: int
    E: int
    K: int
    L: int              # layers in one step
    B: int              # tokens per step (decode) or per layer (prefill)
    steps: int
    mode: int = 0       # 0 softmax-top-K, 1 sigmoid-group
    n_groups: int = 1
    topk_groups: int = 1
    scale: float = 1.0
    eps: float = 1e-20
    S: int = 0          # slots per layer in the pool (0: no pool)
    router: bool = False  # logits from a router GEMV over x (else given fp16 logits)
    zipf: float = 0.0   # popularity bias exponent for given logits
    heads: bool = False
    shared_f: int = 0
    lora_r: int = 0
    lora_alpha_over_r: float = 0.0
    repeat_p: float = 0.0

    @property
    def bundle(self) -> int:
        return gen.bundle_bytes(self.d, self.f)


TINY = Config("tiny", 1001, d=256, f=128, E=16, K=4, L=1, B=8, steps=1, router=True, S=8)
DECODE35 = Config("decode35b", 1002, d=2048, f=512, E=256, K=4, L=40, B=1, steps=256, S=8)
PREFILL35 = Config("prefill35b", 1003, d=2048, f=512, E=256, K=4, L=1, B=2048, steps=1, zipf=1.1)
DECODE8_B1 = Config("decode8b_b1", 1004, d=2048, f=512, E=128, K=8, L=24, B=1, steps=256, mode=1,
                    n_groups=8, topk_groups=4, scale=2.5, router=True, S=16)
DECODE8_B32 = Config("decode8b_b32", 1004, d=2048, f=512, E=128, K=8, L=24, B=32, steps=256, mode=1,
                     n_groups=8, topk_groups=4, scale=2.5, router=True, S=128)
PREROUTED35 = Config("prerouted35b", 1005, d=2048, f=512, E=256, K=4, L=32, B=1, steps=512, S=8,
                     heads=True, shared_f=512, lora_r=16, lora_alpha_over_r=2.0, repeat_p=0.7)

# Chained decode: the 35B stack run as one token through all 40 layers, each
# layer's input the norm of the residual after the previous one; routing given
# per layer (standing in for the staged prediction).
CHAIN35 = Config("chain35b", 1006, d=2048, f=512, E=256, K=4, L=40, B=1, steps=64, S=8)

ALL = {c.name: c for c in (TINY, DECODE35, PREFILL35, DECODE8_B1, DECODE8_B32, PREROUTED35, CHAIN35)}
HEAD_HIDDEN = 512


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases)."""
    vals = {k: getattr(cfg, k) for k in cfg.__dataclass_fields__}
    vals.update(kw)
    return Config(**vals)


# ---------------------------------------------------------------------------
# Per-step inputs
# ---------------------------------------------------------------------------

def activations(cfg: Config, step: int, layer: int, attempt: int = 0) -> np.ndarray:
    """fp16 [B, d] MoE-layer input at (step, layer); N(0,1)."""
    key = gen.stream_key(cfg.seed, gen.TAG_ACT, step, layer, attempt)
    return gen.normal_f16(key, cfg.B * cfg.d).reshape(cfg.B, cfg.d)


def activation_row(cfg: Config, step: int, layer: int, token: int, attempt: int) -> np.ndarray:
    """One redrawn token row (used when a routing decision lacks margin)."""
    key = gen.stream_key(cfg.seed, gen.TAG_REDRAW, gen.TAG_ACT, step, layer, token, attempt)
    return gen.normal_f16(key, cfg.d)


def norm_weight(cfg: Config, layer: int) -> np.ndarray:
    """fp16 [d] norm gain of one layer: 0.2 (1 + 0.1 N(0,1)).

    With these synthetic experts a layer's output grows about quadratically
    with its input; at gain 0.2 each layer adds a few percent to the residual
    (as in trained stacks), where at gain 1 it would add about twice the
    residual and the chain would amplify any rounding difference
    exponentially with depth."""
    z = gen.normal(gen.stream_key(cfg.seed, gen.TAG_NORM, layer), cfg.d)
    return (np.float32(0.2) * (np.float32(1.0) + np.float32(0.1) * z)).astype(np.float16)


def residual0(cfg: Config, step: int) -> np.ndarray:
    """fp32 [d] residual stream entering the first layer at a step; N(0,1)."""
    return gen.normal(gen.stream_key(cfg.seed, gen.TAG_RESID, step), cfg.d).astype(np.float32)


def router_weights(cfg: Config, layer: int) -> np.ndarray:
    """fp16 [E, d] router of one layer; N(0, 0.02)."""
    key = gen.stream_key(cfg.seed, gen.TAG_ROUTER, layer)
    return gen.normal_f16(key, cfg.E * cfg.d, std=0.02).reshape(cfg.E, cfg.d)


def popularity_bias(cfg: Config) -> np.ndarray:
    """fp32 [E] additive logit bias -a*ln(rank_e), rank a seeded permutation.

    -a*ln(rank) is the log of a Zipf(a) pmf up to a constant, which neither
    top-K selection nor a softmax sees.
    """
    order = np.argsort(gen.draws(gen.stream_key(cfg.seed, gen.TAG_PERM), cfg.E), kind="stable")
    rank = np.empty(cfg.E, dtype=np.int64)
    rank[order] = np.arange(1, cfg.E + 1)
    return (-cfg.zipf * np.log(rank.astype(np.float64))).astype(np.float32)


def given_logits(cfg: Config, step: int, layer: int) -> np.ndarray:
    """fp16 [B, E] logits at (step, layer): N(0,1), plus the popularity bias if any."""
    key = gen.stream_key(cfg.seed, gen.TAG_LOGITS, step, layer)
    z = gen.normal(key, cfg.B * cfg.E).reshape(cfg.B, cfg.E)
    if cfg.zipf:
        z = popularity_bias(cfg)[None, :] + z
    return z.astype(np.float16)


# ---------------------------------------------------------------------------
# Prerouted pipeline: heads, shared expert, LoRA, planted hiddens
# ---------------------------------------------------------------------------

@dataclass
class Head:
    fc1_w: np.ndarray   # fp16 [512, d + 2E]
    fc1_b: np.ndarray   # fp16 [512]
    fc2_w: np.ndarray   # fp16 [E, 512]
    fc2_b: np.ndarray   # fp16 [E]
    lin_w: np.ndarray   # fp16 [E, d] linear residual (= consumer layer's router)


def head(cfg: Config, j: int) -> Head:
    """Head j: owned by staged layer j-1, predicts staged layer j one token ahead."""
    din = cfg.d + 2 * cfg.E
    k = lambda t: gen.stream_key(cfg.seed, gen.TAG_HEAD, j, t)
    return Head(
        fc1_w=gen.normal_f16(k(0), HEAD_HIDDEN * din, 0.02).reshape(HEAD_HIDDEN, din),
        fc1_b=gen.normal_f16(k(1), HEAD_HIDDEN, 0.02),
        fc2_w=gen.normal_f16(k(2), cfg.E * HEAD_HIDDEN, 0.02).reshape(cfg.E, HEAD_HIDDEN),
        fc2_b=gen.normal_f16(k(3), cfg.E, 0.02),
        lin_w=router_weights(cfg, j),
    )


def shared_expert(cfg: Config, layer: int):
    """Shared expert of one layer: int4 g64 [(q,s,b)] * 3 with width shared_f."""
    return gen.expert(cfg.seed, layer, 0, cfg.d, cfg.shared_f, tag=gen.TAG_SHARED)


def lora(cfg: Config, layer: int):
    """[(A fp16 [r, in], B fp16 [out, r])] for gate, up, down of the shared expert."""
    out = []
    for p in range(3):
        din, dout = (cfg.d, cfg.shared_f) if p < 2 else (cfg.shared_f, cfg.d)
        a = gen.normal_f16(gen.stream_key(cfg.seed, gen.TAG_LORA, layer, p, 0), cfg.lora_r * din, 0.02)
        b = gen.normal_f16(gen.stream_key(cfg.seed, gen.TAG_LORA, layer, p, 1), dout * cfg.lora_r, 0.02)
        out.append((a.reshape(cfg.lora_r, din), b.reshape(dout, cfg.lora_r)))
    return out


def initial_set(cfg: Config, owner: int) -> np.ndarray:
    """Distinct K experts, uniform: the routing at step 0 of ``owner`` (-1 = unstaged)."""
    d = gen.draws(gen.stream_key(cfg.seed, gen.TAG_TARGETS, 0xFFFF, owner + 1), cfg.E)
    return np.argsort(d, kind="stable")[:cfg.K].astype(np.int32)


def next_set(cfg: Config, prev: np.ndarray, step: int, owner: int) -> np.ndarray:
    """Temporally correlated successor of ``prev``: each member kept with prob
    repeat_p (in place), the others replaced by uniform distinct experts not
    already in the set."""
    d = gen.draws(gen.stream_key(cfg.seed, gen.TAG_TARGETS, step, owner + 1), cfg.K + 4 * cfg.E)
    keep = gen.uniform24(d[:cfg.K]) < np.float32(cfg.repeat_p)
    out = prev.copy()
    taken = set(int(e) for e, kp in zip(prev, keep) if kp)
    pool = d[cfg.K:]
    c = 0
    for k in range(cfg.K):
        if keep[k]:
            continue
        while True:
            e = int(pool[c] % np.uint64(cfg.E))
            c += 1
            if e not in taken and e not in set(int(x) for x in prev):
                break
        taken.add(e)
        out[k] = e
    return out


class Planter:
    """Builds hidden states h so that the head's linear residual lin_w @ h puts
    the planted targets on top: lin_w h = z with z = +8, +7.5, +7, +6.5 at the
    targets (in order) and N(0,1) elsewhere; h = A z + (n - A lin_w n) with
    A = lin_w^T (lin_w lin_w^T)^-1 and n ~ N(0,1) (the null-space part)."""

    def __init__(self, lin_w: np.ndarray):
        w = lin_w.astype(np.float64)
        self.w = w
        self.a = w.T @ np.linalg.inv(w @ w.T)

    def hidden(self, cfg: Config, targets: np.ndarray, step: int, head_j: int, attempt: int = 0) -> np.ndarray:
        kz = gen.stream_key(cfg.seed, gen.TAG_REDRAW, 1, step, head_j, attempt)
        kn = gen.stream_key(cfg.seed, gen.TAG_REDRAW, 2, step, head_j, attempt)
        z = gen.normal(kz, cfg.E).astype(np.float64)
        for i, e in enumerate(targets):
            z[int(e)] = 8.0 - 0.5 * i
        n = gen.normal(kn, cfg.d).astype(np.float64)
        h = self.a @ z + (n - self.a @ (self.w @ n))
        return h.astype(np.float16)


# ---------------------------------------------------------------------------
# Closed forms of the byte counts (pinned by tests against the pages' numbers)
# ---------------------------------------------------------------------------

def expert_bytes(d: int, f: int) -> int:
    return 3 * (d * f // 2 + d * f // gen.GROUP * 4)


def head_weight_bytes(cfg: Config) -> int:
    """Algorithmic bytes one head reads when the K-hot columns are gathered:
    fc1 hidden columns + 2K gathered columns + fc2 + linear residual (fp16)."""
    return 2 * (HEAD_HIDDEN * cfg.d + HEAD_HIDDEN * 2 * cfg.K + cfg.E * HEAD_HIDDEN + cfg.E * cfg.d)


def gib(x: float) -> float:
    return x / float(1 << 30)



# ---------------------------------------------------------------------------
# Prerouted pipeline inputs (32 staged layers, one head per staged layer)
# ---------------------------------------------------------------------------

@dataclass
class Prerouted:
    """Per-step inputs of the prerouted pipeline.

    hin[t]    fp16 [L+1][d]: row 0 is the hidden of the unstaged layer that
              owns head 0; row 1 + l is the MoE input of staged layer l at
              step t. Head j reads row j (its owner's hidden: staged layer
              j-1, or the unstaged owner for j = 0); the decode reads rows
              1..L. Rows 0..L-1 are planted for the targets of step t+1; row L
              (the last staged layer, whose head has no staged consumer) is
              N(0,1).
    owner0[t] int32 [K]: routing of the unstaged owner at step t (p-repeat process).
    r0        int32 [L][K]: routing of the staged layers at step 0.
    targets[t] int32 [L][K]: the sets planted for step t+1.
    """
    hin: np.ndarray
    owner0: np.ndarray
    r0: np.ndarray
    targets: np.ndarray


def prerouted_inputs(cfg: Config, steps: int, accept=None) -> Prerouted:
    """Draw the prerouted pipeline's inputs for `steps` steps.

    accept(t, j, h) -> bool, if given, may reject a planted hidden (the caller
    decides, e.g. on a decision margin); it is then redrawn with the next
    attempt number."""
    L, K = cfg.L, cfg.K
    planters = [Planter(router_weights(cfg, j)) for j in range(L)]
    r0 = np.stack([initial_set(cfg, l) for l in range(L)])
    owner0 = np.empty((steps, K), np.int32)
    owner0[0] = initial_set(cfg, -1)
    for t in range(1, steps):
        owner0[t] = next_set(cfg, owner0[t - 1], t, -1)
    targets = np.empty((steps, L, K), np.int32)
    cur = r0.copy()
    hin = np.empty((steps, L + 1, cfg.d), np.float16)
    for t in range(steps):
        for j in range(L):
            tgt = next_set(cfg, cur[j], t + 1, j)
            targets[t, j] = tgt
            att = 0
            h = planters[j].hidden(cfg, tgt, t, j, att)
            while accept is not None and not accept(t, j, h):
                att += 1
                h = planters[j].hidden(cfg, tgt, t, j, att)
            hin[t, j] = h
        hin[t, L] = activations(cfg, t, L - 1)[0]
        cur = targets[t]
    return Prerouted(hin=hin, owner0=owner0, r0=r0, targets=targets)
