"""C ABI: the library loads, exports every declared symbol, and rejects bad
arguments on the host before touching the GPU (no kernel is launched by any
case here: each one fails validation)."""
import ctypes as C
import os
import re

import pytest

from int4_gather_swiglu_amd import _lib as E

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _declared():
    src = open(os.path.join(ROOT, "include", "e0.h")).read()
    return sorted(set(re.findall(r"^\s*(?:e0_status|int32_t|const char \*|size_t)\s*\n?\s*(e0_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol():
    L = E.lib()
    names = _declared()
    assert set(names) == set(E.EXPORTS), names
    for n in names:
        assert hasattr(L, n)


def test_version_and_strings():
    assert E.abi_version() == 1
    assert E.status_string(0) == "ok"
    assert "workspace" in E.status_string(E.E0_ERR_CAPACITY)
    assert E.status_string(99) == "unknown status"


def test_workspace_sizes():
    dims = E.moe_dims(2048, 512, 256, 4)
    assert E.workspace_bytes(E.E0_OP_ROUTE, dims, 10) == 0
    assert E.workspace_bytes(E.E0_OP_STAGED_DECODE, dims, 40, 1, 0) >= 40 * 5 * 512 * 4
    assert E.workspace_bytes(E.E0_OP_SLOT_UPDATE, dims, 40, 1, 8) > 0
    assert E.workspace_bytes(E.E0_OP_STAGED_DECODE, dims, 40, 0, 0) == 0
    assert E.workspace_bytes(99, dims, 1) == 0


def _route(params, L=1, T=1, Ex=16, logits=FAKE, fp16=0, x=None, wr=None, d=0, idx=FAKE, w=FAKE, lo=None):
    return E.lib().e0_route(C.byref(params), L, T, Ex, C.c_void_p(logits) if logits else None, fp16,
                            C.c_void_p(x) if x else None, C.c_void_p(wr) if wr else None, d,
                            C.c_void_p(idx) if idx else None, C.c_void_p(w) if w else None,
                            C.c_void_p(lo) if lo else None, None)


def test_route_validation():
    assert E.lib().e0_route(None, 1, 1, 16, None, 0, None, None, 0, None, None, None, None) == E.E0_ERR_INVALID_ARG
    assert _route(E.route_params(2, 4)) == E.E0_ERR_INVALID_ARG              # bad mode
    assert _route(E.route_params(0, 17), Ex=16) == E.E0_ERR_UNSUPPORTED_SHAPE  # K > E
    assert _route(E.route_params(0, 4), Ex=2048) == E.E0_ERR_UNSUPPORTED_SHAPE
    assert _route(E.route_params(1, 4, 3, 2, 2.5), Ex=16) == E.E0_ERR_UNSUPPORTED_SHAPE  # groups do not divide E
    assert _route(E.route_params(1, 9, 8, 4, 2.5), Ex=16) == E.E0_ERR_UNSUPPORTED_SHAPE  # K > kept experts
    assert _route(E.route_params(0, 4), idx=None) == E.E0_ERR_INVALID_ARG
    # router path: logits_out required, d a multiple of 64
    assert _route(E.route_params(0, 4), logits=None, x=FAKE, wr=FAKE, d=256) == E.E0_ERR_INVALID_ARG
    assert _route(E.route_params(0, 4), logits=None, x=FAKE, wr=FAKE, d=100, lo=FAKE) == E.E0_ERR_UNSUPPORTED_SHAPE


def _stack(addr=FAKE, stride=1 << 20):
    st = E.Stack()
    for i in range(9):
        st.part[i] = E.Part(addr + 4096 * i, stride, 0)
    return st


def _decode(dims, L=1, B=1, S=8, ws_bytes=1 << 30, pool=None, shared=None, x=FAKE, err=FAKE):
    pool = pool or _stack()
    return E.lib().e0_moe_staged_decode(C.byref(dims), L, B, C.c_void_p(x) if x else None, C.c_void_p(FAKE),
                                        C.c_void_p(FAKE), C.c_void_p(FAKE), S, C.byref(pool),
                                        C.byref(shared) if shared else None, C.c_void_p(FAKE),
                                        C.c_void_p(FAKE), ws_bytes, C.c_void_p(err) if err else None, None)


def test_decode_validation():
    assert _decode(E.moe_dims(100, 512, 256, 4)) == E.E0_ERR_UNSUPPORTED_SHAPE      # d % 64
    assert _decode(E.moe_dims(2048, 96, 256, 4)) == E.E0_ERR_UNSUPPORTED_SHAPE      # f % 64 ok, not supported width
    assert _decode(E.moe_dims(2048, 512, 4, 8)) == E.E0_ERR_UNSUPPORTED_SHAPE       # K > E
    assert _decode(E.moe_dims(2048, 512, 256, 4), B=65) == E.E0_ERR_CAPACITY         # B limit
    assert _decode(E.moe_dims(2048, 512, 256, 4), ws_bytes=16) == E.E0_ERR_CAPACITY  # workspace
    assert _decode(E.moe_dims(2048, 512, 256, 4), x=None) == E.E0_ERR_INVALID_ARG
    assert _decode(E.moe_dims(2048, 512, 256, 4), err=None) == E.E0_ERR_INVALID_ARG
    assert _decode(E.moe_dims(2048, 512, 256, 4), pool=_stack(FAKE + 4)) == E.E0_ERR_INVALID_ARG  # misaligned
    sh = E.Shared()
    sh.w = _stack()
    sh.d_ff = 256
    assert _decode(E.moe_dims(2048, 512, 256, 4), shared=sh) == E.E0_ERR_UNSUPPORTED_SHAPE  # shared width differs
    sh.d_ff = 512
    sh.lora_rank = 64
    assert _decode(E.moe_dims(2048, 512, 256, 4), shared=sh) == E.E0_ERR_UNSUPPORTED_SHAPE


def test_slot_update_validation():
    dims = E.moe_dims(2048, 512, 256, 4)
    L = E.lib()
    ok_stack = _stack()

    def call(dims=dims, S=8, ws_bytes=1 << 20, nxt=FAKE, store=ok_stack):
        return L.e0_slot_update(C.byref(dims), 1, 1, S, C.c_void_p(nxt) if nxt else None, None, C.c_void_p(FAKE),
                                C.c_void_p(FAKE), C.byref(store), C.byref(ok_stack), None, C.c_void_p(FAKE),
                                ws_bytes, C.c_void_p(FAKE), None)
    assert call(S=0) == E.E0_ERR_INVALID_ARG
    assert call(S=5000) == E.E0_ERR_CAPACITY
    assert call(ws_bytes=8) == E.E0_ERR_CAPACITY
    assert call(nxt=None) == E.E0_ERR_INVALID_ARG
    assert call(store=_stack(FAKE + 8)) == E.E0_ERR_INVALID_ARG
    assert call(dims=E.moe_dims(2048, 500, 256, 4)) == E.E0_ERR_UNSUPPORTED_SHAPE


def test_prerouter_validation():
    heads = E.PrerouterHeads(FAKE, 0, None, 0, FAKE, 0, None, 0, FAKE, 0, 512, 0)
    L = E.lib()

    def call(heads=heads, B=1, d=2048, Ex=256, ws_bytes=1 << 24, p=E.route_params(0, 4)):
        return L.e0_prerouter(C.byref(heads), 32, B, d, Ex, C.c_void_p(FAKE), C.c_void_p(FAKE), None, C.byref(p),
                              C.c_void_p(FAKE), C.c_void_p(FAKE), None, C.c_void_p(FAKE), ws_bytes, None)
    assert call(B=65) == E.E0_ERR_CAPACITY
    assert call(d=100) == E.E0_ERR_UNSUPPORTED_SHAPE
    assert call(ws_bytes=16) == E.E0_ERR_CAPACITY
    bad = E.PrerouterHeads(FAKE, 0, None, 0, FAKE, 0, None, 0, FAKE, 0, 100, 0)
    assert call(heads=bad) == E.E0_ERR_UNSUPPORTED_SHAPE
    assert call(p=E.route_params(0, 300)) == E.E0_ERR_UNSUPPORTED_SHAPE


def test_prefill_validation():
    L = E.lib()
    st = _stack()
    dims = E.moe_dims(2048, 100, 256, 4)
    rc = L.e0_moe_sorted_prefill(C.byref(dims), 16, C.c_void_p(FAKE), C.c_void_p(FAKE), C.c_void_p(FAKE),
                                 C.byref(st), C.c_void_p(FAKE), C.c_void_p(FAKE), 1 << 20, C.c_void_p(FAKE), None)
    assert rc == E.E0_ERR_UNSUPPORTED_SHAPE


def test_lora_merge_validation():
    L = E.lib()
    F = C.c_void_p(FAKE)
    G = C.c_void_p(FAKE + 0x100000)  # distinct, non-overlapping fake ranges for the outputs
    H = C.c_void_p(FAKE + 0x200000)
    I = C.c_void_p(FAKE + 0x300000)
    call = L.e0_lora_merge_requant
    # rows not a multiple of 8, cols not a multiple of 64, rank out of range
    assert call(12, 128, F, F, F, F, F, 16, C.c_float(2.0), G, H, I, None) == E.E0_ERR_UNSUPPORTED_SHAPE
    assert call(16, 100, F, F, F, F, F, 16, C.c_float(2.0), G, H, I, None) == E.E0_ERR_UNSUPPORTED_SHAPE
    assert call(16, 128, F, F, F, F, F, 0, C.c_float(2.0), G, H, I, None) == E.E0_ERR_UNSUPPORTED_SHAPE
    assert call(16, 128, F, F, F, F, F, 65, C.c_float(2.0), G, H, I, None) == E.E0_ERR_UNSUPPORTED_SHAPE
    # null, misaligned, non-finite scale, output overlapping an input
    assert call(16, 128, None, F, F, F, F, 16, C.c_float(2.0), G, H, I, None) == E.E0_ERR_INVALID_ARG
    assert call(16, 128, C.c_void_p(FAKE + 2), F, F, F, F, 16, C.c_float(2.0), G, H, I, None) == E.E0_ERR_INVALID_ARG
    assert call(16, 128, F, F, F, F, F, 16, C.c_float(float("nan")), G, H, I, None) == E.E0_ERR_INVALID_ARG
    assert call(16, 128, F, F, F, F, F, 16, C.c_float(2.0), F, H, I, None) == E.E0_ERR_INVALID_ARG


def test_slot_update_lru_validation():
    L = E.lib()
    st = _stack()
    dims = E.moe_dims(2048, 512, 256, 4)
    F = C.c_void_p(FAKE)
    # null last_use, negative step: refused before anything else is read
    assert L.e0_slot_update_lru(C.byref(dims), 1, 1, 8, F, None, F, F, None, 0, C.byref(st), C.byref(st), None, F,
                                1 << 20, F, None) == E.E0_ERR_INVALID_ARG
    assert L.e0_slot_update_lru(C.byref(dims), 1, 1, 8, F, None, F, F, F, -1, C.byref(st), C.byref(st), None, F,
                                1 << 20, F, None) == E.E0_ERR_INVALID_ARG
    # the plain update's checks apply too (S above the limit)
    assert L.e0_slot_update_lru(C.byref(dims), 1, 1, 5000, F, None, F, F, F, 0, C.byref(st), C.byref(st), None, F,
                                1 << 20, F, None) == E.E0_ERR_CAPACITY


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    monkeypatch.setattr(E, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(E, "_LIB", None)
    with pytest.raises(RuntimeError, match="not built"):
        E.lib()


def test_structs_keep_their_tensors_alive():
    # The structs hold raw pointers; the helpers that build them from tensors
    # keep those tensors referenced, so a caller that drops its own names (a
    # set-up function returning only the struct) cannot free memory the
    # library will later read.
    import gc
    import weakref

    import torch
    t = [torch.zeros((2, 8, 16), dtype=torch.int16) for _ in range(5)]
    refs = [weakref.ref(x) for x in t]
    hd = E.heads_from_tensors(*t)
    st_t = torch.zeros((2, E.bundle_bytes(256, 128)), dtype=torch.uint8)
    st_ref = weakref.ref(st_t)
    st = E.stack_from_bundles(st_t, 256, 128, E.bundle_bytes(256, 128))
    la = [torch.zeros((2, 4, 256), dtype=torch.int16) for _ in range(3)]
    lb = [torch.zeros((2, 256, 4), dtype=torch.int16) for _ in range(3)]
    lr = [weakref.ref(x) for x in la + lb]
    sh_t = torch.zeros((2, E.bundle_bytes(256, 128)), dtype=torch.uint8)
    sh_ref = weakref.ref(sh_t)
    sh = E.shared_from_tensors(sh_t, 256, 128, la, lb, 2.0)
    del t, st_t, la, lb, sh_t
    gc.collect()
    assert all(r() is not None for r in refs + lr) and st_ref() is not None and sh_ref() is not None
    del hd, st, sh
    gc.collect()
    assert all(r() is None for r in refs + lr) and st_ref() is None and sh_ref() is None


def test_noalloc_decode_refuses_sizes_beyond_its_array():
    # A decode whose workspace exceeds the fixed array is refused on the host,
    # before the device is touched (pointers are never dereferenced).
    L = E.lib()
    dims = E.moe_dims(2048, 2048, 1024, 8)
    need = E.workspace_bytes(E.E0_OP_STAGED_DECODE, dims, 64, 64, 0)
    assert need > E.E0_NOALLOC_SCRATCH_BYTES
    st = E.stack_from_bundles(FAKE, 2048, 2048, 1 << 20)
    rc = L.e0_moe_staged_decode_noalloc(C.byref(dims), 64, 64, FAKE, FAKE, FAKE, FAKE, 128, C.byref(st), None,
                                        FAKE, FAKE, None)
    assert rc == E.E0_ERR_CAPACITY
    assert L.e0_moe_staged_decode_noalloc(None, 1, 1, FAKE, FAKE, FAKE, FAKE, 8, C.byref(st), None, FAKE, FAKE,
                                          None) == E.E0_ERR_INVALID_ARG
