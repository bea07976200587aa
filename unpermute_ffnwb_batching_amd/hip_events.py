"""Minimal HIP events for the library's timing hooks and the unpermute's auxiliary-stream
fork and join (plumbing only).

The descriptors' ev_* fields take hipEvent_t handles, which the library binds to the
timed kernel's launch (or records on the stream under graph capture).  These events are
created with hipEventDisableSystemFence: completing them issues no system-scope release,
so timing a kernel inside a sequence of launches does not stall the stream.
"""

import ctypes

import torch  # noqa: F401  (loads the HIP runtime first)

_HIP = None
HIP_EVENT_DISABLE_TIMING = 0x2
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _hip():
    global _HIP
    if _HIP is None:
        h = ctypes.CDLL("libamdhip64.so.7")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        for f in ("hipEventCreateWithFlags", "hipEventDestroy", "hipEventElapsedTime", "hipEventSynchronize",
                  "hipEventRecord"):
            getattr(h, f).restype = ctypes.c_int
        _HIP = h
    return _HIP


class HipEvent:
    """A hipEvent_t usable as a timing hook (``.handle``) and with elapsed-time queries."""

    def __init__(self, flags=HIP_EVENT_DISABLE_SYSTEM_FENCE):
        self.handle = ctypes.c_void_p()
        st = _hip().hipEventCreateWithFlags(ctypes.byref(self.handle), flags)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        st = _hip().hipEventRecord(self.handle, ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def synchronize(self):
        _hip().hipEventSynchronize(self.handle)

    def elapsed_ms(self, end):
        ms = ctypes.c_float(0.0)
        st = _hip().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if _HIP is not None and self.handle:
            _HIP.hipEventDestroy(self.handle)
            self.handle = ctypes.c_void_p()
