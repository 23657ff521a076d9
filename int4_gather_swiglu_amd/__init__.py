"""MI355X (gfx950) routed-expert int4 group-64 SwiGLU hot path.

The kernels live in libe0.so (C ABI: include/e0.h); ``_lib`` is the ctypes
binding with the same call names. Build with ``__graft_entry__.build()``.
"""
from . import _lib  # noqa: F401
from ._lib import (E0Error, e0_moe_sorted_prefill, e0_moe_staged_decode, e0_prerouter, e0_route,  # noqa: F401
                   e0_slot_update)
