"""HIP events with explicit fence flags, for the step pipeline and for kernel timing.

torch's events always record with a system-scope release: the GPU writes back and invalidates its caches when the
event completes, which costs the work after it a few microseconds. Two uses here do not need that fence:

- an event that only orders a later copy after kernels that READ a buffer (write-after-read): the copy engine's
  writes cannot be affected by what the kernels cached;
- a pair of events that only time the kernels between them.

Both are created with hipEventDisableSystemFence. Events that publish data to a consumer (the copy of the step's
metadata that the kernels then read) keep the default fence.

The calls go to the HIP runtime that torch has loaded (one runtime per process), with torch streams' raw handles.
The step pipeline also enqueues its per-step metadata copy here (`memcpy_h2d_async`): one runtime call instead of
torch's stream context and tensor copy, whose host cost is a tenth of a small step.
"""
from __future__ import annotations

import ctypes as C
import os

HIP_MEMCPY_HOST_TO_DEVICE = 1
HIP_EVENT_DISABLE_TIMING = 0x2
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

_hip = None


def _runtime():
    global _hip
    if _hip is None:
        import torch
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        lib = C.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")
        lib.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        lib.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        lib.hipStreamWaitEvent.argtypes = [C.c_void_p, C.c_void_p, C.c_uint]
        lib.hipEventSynchronize.argtypes = [C.c_void_p]
        lib.hipEventQuery.argtypes = [C.c_void_p]
        lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        lib.hipEventDestroy.argtypes = [C.c_void_p]
        lib.hipMemcpyAsync.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
        _hip = lib
    return _hip


def _check(err: int, what: str) -> None:
    if err != 0:
        raise RuntimeError(f"{what} failed with HIP error {err}")


def memcpy_h2d_async(dst: int, src: int, nbytes: int, stream: C.c_void_p) -> None:
    """Enqueue a copy of nbytes from pinned host address src to device address dst on the raw stream handle."""
    _check(_runtime().hipMemcpyAsync(dst, src, nbytes, HIP_MEMCPY_HOST_TO_DEVICE, stream), "hipMemcpyAsync")


class HipEvent:
    """One HIP event. timing=True keeps timestamps (for elapsed_time); system_fence=False records without the
    system-scope release (see the module docstring for when that is safe)."""

    def __init__(self, timing: bool = False, system_fence: bool = True):
        self._lib = _runtime()
        flags = 0 if timing else HIP_EVENT_DISABLE_TIMING
        if not system_fence:
            flags |= HIP_EVENT_DISABLE_SYSTEM_FENCE
        self.handle = C.c_void_p()
        _check(self._lib.hipEventCreateWithFlags(C.byref(self.handle), flags), "hipEventCreateWithFlags")

    def record(self, stream) -> None:
        """Record on a torch stream."""
        _check(self._lib.hipEventRecord(self.handle, C.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def wait(self, stream) -> None:
        """Make a torch stream wait for this event's last record."""
        _check(self._lib.hipStreamWaitEvent(C.c_void_p(stream.cuda_stream), self.handle, 0), "hipStreamWaitEvent")

    def record_on(self, handle: C.c_void_p) -> None:
        """Record on a raw stream handle."""
        _check(self._lib.hipEventRecord(self.handle, handle), "hipEventRecord")

    def wait_on(self, handle: C.c_void_p) -> None:
        """Make the stream with this raw handle wait for this event's last record."""
        _check(self._lib.hipStreamWaitEvent(handle, self.handle, 0), "hipStreamWaitEvent")

    def synchronize(self) -> None:
        _check(self._lib.hipEventSynchronize(self.handle), "hipEventSynchronize")

    def query(self) -> bool:
        return self._lib.hipEventQuery(self.handle) == 0

    def elapsed_time(self, end: "HipEvent") -> float:
        """Milliseconds from this event to `end` (both created with timing=True and completed)."""
        ms = C.c_float()
        _check(self._lib.hipEventElapsedTime(C.byref(ms), self.handle, end.handle), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        lib, h = getattr(self, "_lib", None), getattr(self, "handle", None)
        if lib is not None and h is not None and h.value:
            lib.hipEventDestroy(h)
            self.handle = None
