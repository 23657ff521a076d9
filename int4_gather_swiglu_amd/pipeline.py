"""Staged decode pipeline: the C-ABI calls of one decode step, sequenced on
HIP streams. Holds device buffers; computes nothing itself.

Per step t (fixed double-buffered slots, routing ids kept on the GPU; the
update for step t+1 overlaps step t: koala.ai.kr paths table and Fig. 1
timeline; jaehun.me review, report 3.1):

  side : waits for main's decode of step t-1 (it read idx[(t+1) % 2] and the
         slots the update may rewrite), not for main's wait on the side
  side : routing of step t+1          -> idx[(t+1) % 2]   (e0_route)
  side : slot update                  next = idx[(t+1) % 2], in use = idx[t % 2]
  main : staged decode of step t      reads idx[t % 2] through the slot table
  main : (before step t+1) waits for the side stream

With the prerouter, the routing of step t+1 is the heads' prediction made at
step t (one flush for all staged layers, then the slot update; koala.ai.kr
prerouter section): PrerouterPipeline. With the one-token lead, the heads of
step t and the slot update for step t+1 can run on the side stream while
the main stream decodes step t (predict(..., on_side=True)).

The update only writes slots whose experts are in neither set, and leaves the
slot-table entries of step t's experts untouched, so it can run while step t
reads the pool.
"""
from __future__ import annotations

import torch

from . import _lib as E
from .streams import Event


class StagedPipeline:
    def __init__(self, dims: E.MoeDims, L: int, B: int, S: int, store: E.Stack, pool: E.Stack,
                 shared: E.Shared | None = None, device="cuda", side_stream: bool = True, hot_set: bool = False):
        """hot_set: keep the S slots per layer as a least-recently-used hot set of
        the store (e0_slot_update_lru) instead of the lowest-free-slot rule."""
        self.dims, self.L, self.B, self.S = dims, L, B, S
        self.hot_set = hot_set
        self.step = 0
        self.store, self.pool, self.shared = store, pool, shared
        K, Ex = dims.top_k, dims.n_experts
        dev = torch.device(device)
        self.dev = dev
        self.slot_of = torch.full((L, Ex), -1, dtype=torch.int32, device=dev)
        self.expert_of = torch.full((L, S), -1, dtype=torch.int32, device=dev)
        self.last_use = torch.full((L, S), -1, dtype=torch.int32, device=dev)
        self.idx = torch.zeros((2, L, B, K), dtype=torch.int32, device=dev)
        self.w = torch.zeros((2, L, B, K), dtype=torch.float32, device=dev)
        self.n_copied = torch.zeros((L,), dtype=torch.int32, device=dev)
        self.err = torch.zeros((1,), dtype=torch.int32, device=dev)
        r = shared.lora_rank if shared is not None else 0
        self.ws_dec = torch.empty(E.workspace_bytes(E.E0_OP_STAGED_DECODE, dims, L, B, r), dtype=torch.uint8,
                                  device=dev)
        self.ws_slot = torch.empty(E.workspace_bytes(E.E0_OP_SLOT_UPDATE, dims, L, B, S), dtype=torch.uint8,
                                   device=dev)
        self.main = torch.cuda.current_stream(dev)
        self.side = torch.cuda.Stream(dev) if side_stream else self.main
        self.ev_routed = Event()
        self.ev_updated = Event()
        self.ev_decoded = Event()  # recorded on main right after each decode
        self._decoded = False

    # -- pieces -------------------------------------------------------------
    def side_after_main(self):
        """Make the side stream wait for everything enqueued on main so far
        (nothing to do when both are one stream)."""
        if self.side is not self.main:
            self.ev_routed.record(self.main)
            self.ev_routed.wait(self.side)

    def side_after_decode(self):
        """Make the side stream wait for main's work up to the last
        mark_decoded (a decode), not for what main enqueued after it, such as
        its wait for the side stream's last update: the next update's plan and
        copies only need the decode of the step before the one in flight to
        have finished."""
        if self.side is not self.main and self._decoded:
            self.ev_decoded.wait(self.side)

    def mark_decoded(self):
        """Record main's work so far (a decode, and whatever the caller put on
        main after it that must also precede the next update) as what the next
        side_after_decode waits for."""
        if self.side is not self.main:
            self.ev_decoded.record(self.main)
            self._decoded = True

    def route_given(self, buf: int, params: E.RouteParams, logits, fp16: bool = True, on_side: bool = False):
        """Route step logits [L][B][E] (fp16 bits or fp32) into idx/w[buf]."""
        E.e0_route(params, self.L, self.B, self.dims.n_experts, logits, fp16, None, None, 0, self.idx[buf],
                   self.w[buf], None, stream=self.side if on_side else self.main)

    def route_router(self, buf: int, params: E.RouteParams, x, w_router, logits_out, on_side: bool = False):
        """Route with each layer's own router over x [L][B][d]."""
        E.e0_route(params, self.L, self.B, self.dims.n_experts, None, False, x, w_router, self.dims.d_model,
                   self.idx[buf], self.w[buf], logits_out, stream=self.side if on_side else self.main)

    def update_ids(self, nxt, cur, after_main: bool = True, after_decode: bool = False):
        """Slot update for routing ids `nxt` [L][B][K], protecting `cur` (or
        None), on the side stream: after everything enqueued on main so far
        (after_main), or after main's last decode only (after_decode)."""
        if after_decode:
            self.side_after_decode()
        elif after_main:
            self.side_after_main()
        if self.hot_set:
            E.e0_slot_update_lru(self.dims, self.L, self.B, self.S, nxt, cur, self.slot_of, self.expert_of,
                                 self.last_use, self.step, self.store, self.pool, self.n_copied, self.ws_slot,
                                 self.err, stream=self.side)
            self.step += 1
        else:
            E.e0_slot_update(self.dims, self.L, self.B, self.S, nxt, cur, self.slot_of, self.expert_of, self.store,
                             self.pool, self.n_copied, self.ws_slot, self.err, stream=self.side)
        if self.side is not self.main:
            self.ev_updated.record(self.side)

    def update(self, nxt: int, cur: int | None, after_main: bool = True):
        """Slot update for idx[nxt], protecting idx[cur], on the side stream
        (after the work on main unless after_main is False)."""
        self.update_ids(self.idx[nxt], None if cur is None else self.idx[cur], after_main)

    def join(self):
        """Make main wait for the last slot update on the side stream."""
        if self.side is not self.main:
            self.ev_updated.wait(self.main)

    def decode_ids(self, idx, w, x, y):
        E.e0_moe_staged_decode(self.dims, self.L, self.B, x, idx, w, self.slot_of, self.S, self.pool, self.shared, y,
                               self.ws_dec, self.err, stream=self.main)

    def decode(self, buf: int, x, y):
        self.decode_ids(self.idx[buf], self.w[buf], x, y)

    def decode_chain(self, buf: int, r_in, norm_w, eps: float, y, r_out):
        """Chained decode of one token through the L layers (batch 1): layer
        l's input is the normed residual after layer l - 1."""
        if getattr(self, "ws_chain", None) is None:
            n = E.workspace_bytes(E.E0_OP_CHAINED_DECODE, self.dims, self.L)
            if n == 0:
                raise E.E0Error(E.E0_ERR_UNSUPPORTED_SHAPE, "e0_moe_chained_decode")
            self.ws_chain = torch.empty(n, dtype=torch.uint8, device=self.dev)
        E.e0_moe_chained_decode(self.dims, self.L, r_in, norm_w, eps, self.idx[buf], self.w[buf], self.slot_of, self.S,
                                self.pool, y, r_out, self.ws_chain, self.err, stream=self.main)


class PrerouterPipeline(StagedPipeline):
    """Staged decode whose routing is the prerouter heads' prediction.

    Routing state R[t] is [L+1][B][K]: row 0 is the unstaged layer owning head
    0 (given), rows 1..L the staged layers. Head j reads its owner's hidden
    hin[j] (hin: [L+1][B][d], rows 1..L are also the decode's inputs), the
    owner's current and previous routing R[t][j], R[t-1][j], and writes
    R[t+1][j+1]."""

    def __init__(self, dims, L, B, S, store, pool, heads: E.PrerouterHeads, route: E.RouteParams,
                 shared=None, device="cuda", side_stream: bool = True, hot_set: bool = False):
        super().__init__(dims, L, B, S, store, pool, shared, device, side_stream, hot_set)
        self.heads, self.route = heads, route
        hd = E.moe_dims(dims.d_model, heads.hidden, dims.n_experts, dims.top_k)
        self.ws_pre = torch.empty(E.workspace_bytes(E.E0_OP_PREROUTER, hd, L, B), dtype=torch.uint8, device=self.dev)

    def predict(self, hin, r_cur, r_prev, r_next, w_next, logits_out=None, on_side: bool = False):
        """Heads at step t: hin [L+1][B][d], r_cur / r_prev [L+1][B][K] (r_prev
        may be None) -> r_next[1:], w_next[1:] (the routing of step t+1), on the
        main stream or (on_side) the side stream."""
        E.e0_prerouter(self.heads, self.L, self.B, self.dims.d_model, self.dims.n_experts, hin, r_cur, r_prev,
                       self.route, r_next[1:], w_next[1:], logits_out, self.ws_pre,
                       stream=self.side if on_side else self.main)
