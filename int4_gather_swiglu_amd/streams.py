"""HIP events over torch's streams: ordering between the pipeline's two streams,
and timing. Plumbing only (no computation).

torch's events record with a system-scope release, which writes the GPU's
caches back so that host code could read device memory after the event. The
pipeline's events only order kernels of one device on two of its streams, and
timing events only take timestamps, so both are created with the system-scope
fence off (the release and acquire stay device-wide). On the staged decode
step the system-scope fences cost about 4 us of the step for the two ordering
events, and the four timing events of a timed step about 7 us with a
device-scope release against 4 us without the fence.

The HIP runtime is the one torch has loaded (same soname), so the stream
handles torch hands out are valid here."""
from __future__ import annotations

import ctypes as C

import torch  # noqa: F401  (loads the HIP runtime these calls go to)

_HIP_EVENT_DISABLE_TIMING = 0x2
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

_hip = None


def _rt() -> C.CDLL:
    global _hip
    if _hip is None:
        h = C.CDLL("libamdhip64.so.7")
        h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        h.hipEventDestroy.argtypes = [C.c_void_p]
        h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        h.hipStreamWaitEvent.argtypes = [C.c_void_p, C.c_void_p, C.c_uint]
        h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        h.hipEventSynchronize.argtypes = [C.c_void_p]
        for f in (h.hipEventCreateWithFlags, h.hipEventDestroy, h.hipEventRecord, h.hipStreamWaitEvent,
                  h.hipEventElapsedTime, h.hipEventSynchronize):
            f.restype = C.c_int
        _hip = h
    return _hip


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


def _stream(s) -> C.c_void_p:
    return C.c_void_p(s.cuda_stream)


class Event:
    """timing=False: an ordering event (no timestamps); timing=True: a timing
    event. Neither has a system-scope fence."""

    def __init__(self, timing: bool = False):
        self._h = C.c_void_p()
        flags = _HIP_EVENT_DISABLE_SYSTEM_FENCE | (0 if timing else _HIP_EVENT_DISABLE_TIMING)
        _check(_rt().hipEventCreateWithFlags(C.byref(self._h), flags), "hipEventCreateWithFlags")

    def record(self, stream=None):
        """Record on `stream` (torch's current stream if None)."""
        s = torch.cuda.current_stream() if stream is None else stream
        _check(_rt().hipEventRecord(self._h, _stream(s)), "hipEventRecord")

    def wait(self, stream):
        """Make `stream` wait for the work this event recorded."""
        _check(_rt().hipStreamWaitEvent(_stream(stream), self._h, 0), "hipStreamWaitEvent")

    def synchronize(self):
        _check(_rt().hipEventSynchronize(self._h), "hipEventSynchronize")

    def elapsed_time(self, end: "Event") -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = C.c_float()
        _check(_rt().hipEventElapsedTime(C.byref(ms), self._h, end._h), "hipEventElapsedTime")
        return float(ms.value)

    def __del__(self):
        if _hip is not None and self._h:
            _hip.hipEventDestroy(self._h)
            self._h = C.c_void_p()
