"""ctypes binding of libe0 (include/e0.h): argument marshalling only.

Every function takes torch tensors on the GPU (or None where the ABI allows
NULL), passes raw device pointers and the current HIP stream, and raises
E0Error on a nonzero status. All computation happens in the HIP kernels of
libe0.so; there is no fallback: if the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libe0.so")

E0_OK, E0_ERR_INVALID_ARG, E0_ERR_UNSUPPORTED_SHAPE, E0_ERR_CAPACITY, E0_ERR_HIP = range(5)
E0_DEV_BAD_ID, E0_DEV_NOT_RESIDENT, E0_DEV_NO_SLOT = 1, 2, 4
(E0_OP_ROUTE, E0_OP_PREROUTER, E0_OP_STAGED_DECODE, E0_OP_SORTED_PREFILL, E0_OP_SLOT_UPDATE,
 E0_OP_CHAINED_DECODE) = range(6)

E0_NOALLOC_SCRATCH_BYTES = 32 << 20  # size of the fixed workspace of e0_moe_staged_decode_noalloc
EXPORTS = ["e0_abi_version", "e0_status_string", "e0_workspace_bytes", "e0_route", "e0_prerouter",
           "e0_moe_staged_decode", "e0_moe_sorted_prefill", "e0_slot_update", "e0_moe_chained_decode",
           "e0_lora_merge_requant", "e0_slot_update_lru", "e0_moe_staged_decode_noalloc",
           "e0_probe_stream_read", "e0_probe_mfma"]


class E0Error(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {status_string(status)} (status {status})")


class RouteParams(C.Structure):
    _fields_ = [("mode", C.c_int32), ("k", C.c_int32), ("n_groups", C.c_int32), ("topk_groups", C.c_int32),
                ("scale", C.c_float), ("eps", C.c_float)]


class MoeDims(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("d_ff", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32)]


class Part(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("slot_stride", C.c_int64), ("layer_stride", C.c_int64)]


class Stack(C.Structure):
    _fields_ = [("part", Part * 9)]


class Shared(C.Structure):
    _fields_ = [("w", Stack), ("d_ff", C.c_int32), ("lora_rank", C.c_int32), ("lora_scale", C.c_float),
                ("pad_", C.c_int32), ("lora_a", C.c_void_p * 3), ("lora_a_layer_stride", C.c_int64 * 3),
                ("lora_b", C.c_void_p * 3), ("lora_b_layer_stride", C.c_int64 * 3)]


class PrerouterHeads(C.Structure):
    _fields_ = [("fc1_w", C.c_void_p), ("fc1_w_stride", C.c_int64), ("fc1_b", C.c_void_p),
                ("fc1_b_stride", C.c_int64), ("fc2_w", C.c_void_p), ("fc2_w_stride", C.c_int64),
                ("fc2_b", C.c_void_p), ("fc2_b_stride", C.c_int64), ("lin_w", C.c_void_p),
                ("lin_w_stride", C.c_int64), ("hidden", C.c_int32), ("pad_", C.c_int32)]


_LIB = None


def lib() -> C.CDLL:
    """The loaded libe0.so. Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libe0.so not built: run __graft_entry__.build() (expected {LIB_PATH})")
        # torch first: its bundled HIP runtime has the same soname as the
        # system one libe0.so was linked against, so loading torch first makes
        # this library bind to torch's runtime instead of starting a second
        # HIP runtime in the process (which then finds no device).
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        L.e0_abi_version.restype = C.c_int32
        L.e0_status_string.restype = C.c_char_p
        L.e0_status_string.argtypes = [C.c_int32]
        L.e0_workspace_bytes.restype = C.c_size_t
        L.e0_workspace_bytes.argtypes = [C.c_int32, C.POINTER(MoeDims), C.c_int32, C.c_int32, C.c_int32]
        vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.e0_route.argtypes = [C.POINTER(RouteParams), i32, i32, i32, vp, i32, vp, vp, i32, vp, vp, vp, vp]
        L.e0_prerouter.argtypes = [C.POINTER(PrerouterHeads), i32, i32, i32, i32, vp, vp, vp,
                                   C.POINTER(RouteParams), vp, vp, vp, vp, sz, vp]
        L.e0_moe_staged_decode.argtypes = [C.POINTER(MoeDims), i32, i32, vp, vp, vp, vp, i32, C.POINTER(Stack),
                                           C.POINTER(Shared), vp, vp, sz, vp, vp]
        L.e0_moe_sorted_prefill.argtypes = [C.POINTER(MoeDims), i32, vp, vp, vp, C.POINTER(Stack), vp, vp, sz,
                                            vp, vp]
        L.e0_slot_update.argtypes = [C.POINTER(MoeDims), i32, i32, i32, vp, vp, vp, vp, C.POINTER(Stack),
                                     C.POINTER(Stack), vp, vp, sz, vp, vp]
        L.e0_slot_update_lru.argtypes = [C.POINTER(MoeDims), i32, i32, i32, vp, vp, vp, vp, vp, i32, C.POINTER(Stack),
                                     C.POINTER(Stack), vp, vp, sz, vp, vp]
        L.e0_moe_chained_decode.argtypes = [C.POINTER(MoeDims), i32, vp, vp, C.c_float, vp, vp, vp, i32,
                                            C.POINTER(Stack), vp, vp, vp, sz, vp, vp]
        L.e0_lora_merge_requant.argtypes = [i32, i32, vp, vp, vp, vp, vp, i32, C.c_float, vp, vp, vp, vp]
        L.e0_moe_staged_decode_noalloc.argtypes = [C.POINTER(MoeDims), i32, i32, vp, vp, vp, vp, i32,
                                                   C.POINTER(Stack), C.POINTER(Shared), vp, vp, vp]
        L.e0_probe_stream_read.argtypes = [vp, sz, vp, vp]
        L.e0_probe_mfma.argtypes = [i32, i32, vp, C.POINTER(C.c_double), vp]
        for n in ("e0_route", "e0_prerouter", "e0_moe_staged_decode", "e0_moe_sorted_prefill", "e0_slot_update",
                  "e0_moe_chained_decode", "e0_lora_merge_requant", "e0_slot_update_lru",
                  "e0_moe_staged_decode_noalloc", "e0_probe_stream_read", "e0_probe_mfma"):
            getattr(L, n).restype = C.c_int32
        _LIB = L
    return _LIB


def status_string(s: int) -> str:
    return lib().e0_status_string(s).decode()


def abi_version() -> int:
    return lib().e0_abi_version()


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _check(status: int, call: str):
    if status != E0_OK:
        raise E0Error(status, call)


# ---------------------------------------------------------------------------
# Layout helpers (the bundle format of include/e0.h)
# ---------------------------------------------------------------------------

def bundle_part_sizes(d: int, f: int):
    """Bytes of the nine parts of one expert, in e0_stack order."""
    qb = d * f // 2
    sb = d * f // 64 * 2
    return [qb, sb, sb] * 3


def bundle_bytes(d: int, f: int) -> int:
    return sum(bundle_part_sizes(d, f))


def stack_from_bundles(base, d: int, f: int, slot_stride: int, layer_stride: int = 0) -> Stack:
    """e0_stack over bundle-contiguous experts starting at tensor/pointer `base`.
    The returned struct holds a reference to a tensor `base`, so the memory its
    pointers name lives as long as the struct."""
    addr = base if isinstance(base, int) else base.data_ptr()
    st = Stack()
    off = 0
    for i, sz in enumerate(bundle_part_sizes(d, f)):
        st.part[i] = Part(addr + off, slot_stride, layer_stride)
        off += sz
    st._keep = None if isinstance(base, int) else base
    return st


def route_params(mode=0, k=4, n_groups=1, topk_groups=1, scale=1.0, eps=1e-20) -> RouteParams:
    return RouteParams(mode, k, n_groups, topk_groups, scale, eps)


def moe_dims(d_model, d_ff, n_experts, top_k) -> MoeDims:
    return MoeDims(d_model, d_ff, n_experts, top_k)


def workspace_bytes(op: int, dims: MoeDims, n: int, b: int = 1, s: int = 0) -> int:
    return lib().e0_workspace_bytes(op, C.byref(dims), n, b, s)


# ---------------------------------------------------------------------------
# The five calls
# ---------------------------------------------------------------------------

def e0_route(params: RouteParams, n_layers: int, T: int, E: int, logits=None, logits_fp16: bool = False,
             x=None, w_router=None, d: int = 0, idx=None, w=None, logits_out=None, stream=None):
    _check(lib().e0_route(C.byref(params), n_layers, T, E, _ptr(logits), int(bool(logits_fp16)), _ptr(x),
                          _ptr(w_router), d, _ptr(idx), _ptr(w), _ptr(logits_out), _stream(stream)), "e0_route")


def e0_prerouter(heads: PrerouterHeads, n_heads: int, B: int, d: int, E: int, h, cur_idx, prev_idx,
                 params: RouteParams, next_idx, next_w, logits_out, ws, stream=None):
    _check(lib().e0_prerouter(C.byref(heads), n_heads, B, d, E, _ptr(h), _ptr(cur_idx), _ptr(prev_idx),
                              C.byref(params), _ptr(next_idx), _ptr(next_w), _ptr(logits_out), _ptr(ws),
                              ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)),
           "e0_prerouter")


def e0_moe_staged_decode(dims: MoeDims, L: int, B: int, x, idx, w, slot_of, S: int, pool: Stack,
                         shared: Shared | None, y, ws, dev_err, stream=None):
    _check(lib().e0_moe_staged_decode(C.byref(dims), L, B, _ptr(x), _ptr(idx), _ptr(w), _ptr(slot_of), S,
                                      C.byref(pool), C.byref(shared) if shared is not None else None, _ptr(y),
                                      _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                      _ptr(dev_err), _stream(stream)), "e0_moe_staged_decode")


def e0_moe_staged_decode_noalloc(dims: MoeDims, L: int, B: int, x, idx, w, slot_of, S: int, pool: Stack,
                                 shared: Shared | None, y, dev_err, stream=None):
    """The staged decode with the library's own fixed workspace (allocates nothing)."""
    _check(lib().e0_moe_staged_decode_noalloc(C.byref(dims), L, B, _ptr(x), _ptr(idx), _ptr(w), _ptr(slot_of), S,
                                              C.byref(pool), C.byref(shared) if shared is not None else None,
                                              _ptr(y), _ptr(dev_err), _stream(stream)),
           "e0_moe_staged_decode_noalloc")


def e0_moe_chained_decode(dims: MoeDims, L: int, r_in, norm_w, eps: float, idx, w, slot_of, S: int, pool: Stack,
                          y, r_out, ws, dev_err, stream=None):
    _check(lib().e0_moe_chained_decode(C.byref(dims), L, _ptr(r_in), _ptr(norm_w), C.c_float(eps), _ptr(idx),
                                       _ptr(w), _ptr(slot_of), S, C.byref(pool), _ptr(y), _ptr(r_out), _ptr(ws),
                                       ws.numel() * ws.element_size() if ws is not None else 0, _ptr(dev_err),
                                       _stream(stream)), "e0_moe_chained_decode")


def e0_lora_merge_requant(rows: int, cols: int, q, s, b, lora_b, lora_a, r: int, alpha_over_r: float, q_out, s_out,
                          b_out, stream=None):
    _check(lib().e0_lora_merge_requant(rows, cols, _ptr(q), _ptr(s), _ptr(b), _ptr(lora_b), _ptr(lora_a), r,
                                       C.c_float(alpha_over_r), _ptr(q_out), _ptr(s_out), _ptr(b_out),
                                       _stream(stream)), "e0_lora_merge_requant")


def e0_moe_sorted_prefill(dims: MoeDims, T: int, x, idx, w, layer: Stack, y, ws, dev_err, stream=None):
    _check(lib().e0_moe_sorted_prefill(C.byref(dims), T, _ptr(x), _ptr(idx), _ptr(w), C.byref(layer), _ptr(y),
                                       _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                       _ptr(dev_err), _stream(stream)), "e0_moe_sorted_prefill")


def e0_slot_update(dims: MoeDims, L: int, B: int, S: int, next_idx, cur_idx, slot_of, expert_of, store: Stack,
                   pool: Stack, n_copied, ws, dev_err, stream=None):
    _check(lib().e0_slot_update(C.byref(dims), L, B, S, _ptr(next_idx), _ptr(cur_idx), _ptr(slot_of),
                                _ptr(expert_of), C.byref(store), C.byref(pool), _ptr(n_copied), _ptr(ws),
                                ws.numel() * ws.element_size() if ws is not None else 0, _ptr(dev_err),
                                _stream(stream)), "e0_slot_update")


def e0_slot_update_lru(dims: MoeDims, L: int, B: int, S: int, next_idx, cur_idx, slot_of, expert_of, last_use,
                       step: int, store: Stack, pool: Stack, n_copied, ws, dev_err, stream=None):
    _check(lib().e0_slot_update_lru(C.byref(dims), L, B, S, _ptr(next_idx), _ptr(cur_idx), _ptr(slot_of),
                                    _ptr(expert_of), _ptr(last_use), step, C.byref(store), C.byref(pool),
                                    _ptr(n_copied), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                    _ptr(dev_err), _stream(stream)), "e0_slot_update_lru")


def heads_from_tensors(fc1_w, fc1_b, fc2_w, fc2_b, lin_w) -> PrerouterHeads:
    """e0_prerouter_heads over stacked per-head fp16 tensors:
    fc1_w [H][hid][d+2E], fc1_b [H][hid] or None, fc2_w [H][E][hid],
    fc2_b [H][E] or None, lin_w [H][E][d]. The struct holds references to the
    tensors, so the memory its pointers name lives as long as the struct."""
    def ps(t):
        return (t.data_ptr(), t[0].numel() * t.element_size()) if t is not None else (None, 0)
    (a, sa), (b, sb), (c, sc), (d_, sd), (e, se) = ps(fc1_w), ps(fc1_b), ps(fc2_w), ps(fc2_b), ps(lin_w)
    hd = PrerouterHeads(a, sa, b, sb, c, sc, d_, sd, e, se, int(fc1_w.shape[1]), 0)
    hd._keep = (fc1_w, fc1_b, fc2_w, fc2_b, lin_w)
    return hd


def shared_from_tensors(store, d: int, f: int, lora_a=None, lora_b=None, lora_scale: float = 0.0) -> Shared:
    """e0_shared over per-layer bundles store [L][bundle] (one shared expert
    per layer) and optional LoRA: lora_a[p] [L][r][in_p], lora_b[p] [L][out_p][r].
    The struct holds references to the tensors, so the memory its pointers name
    lives as long as the struct."""
    sh = Shared()
    sh._keep = (store, None if lora_a is None else list(lora_a), None if lora_b is None else list(lora_b))
    bb = bundle_bytes(d, f)
    sh.w = stack_from_bundles(store, d, f, bb, store[0].numel() * store.element_size())
    sh.d_ff = f
    sh.lora_rank = int(lora_a[0].shape[1]) if lora_a is not None else 0
    sh.lora_scale = lora_scale
    if lora_a is not None:
        for p in range(3):
            sh.lora_a[p] = lora_a[p].data_ptr()
            sh.lora_a_layer_stride[p] = lora_a[p][0].numel() * lora_a[p].element_size()
            sh.lora_b[p] = lora_b[p].data_ptr()
            sh.lora_b_layer_stride[p] = lora_b[p][0].numel() * lora_b[p].element_size()
    return sh


def e0_probe_stream_read(src, sink, stream=None):
    """One streaming read of the whole device tensor `src` (measurement probe)."""
    _check(lib().e0_probe_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)),
           "e0_probe_stream_read")


def e0_probe_mfma(blocks: int, iters: int, sink, stream=None) -> float:
    """Independent fp16 MFMAs on `blocks` workgroups (measurement probe); returns the launch's FLOP."""
    flop = C.c_double(0.0)
    _check(lib().e0_probe_mfma(blocks, iters, _ptr(sink), C.byref(flop), _stream(stream)), "e0_probe_mfma")
    return flop.value
