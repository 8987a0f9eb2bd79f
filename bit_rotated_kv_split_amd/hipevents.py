"""Raw HIP events through ctypes (libamdhip64), for timing a kernel that the
library launches between other kernels on the same stream."""
from __future__ import annotations

import ctypes

_hip = None


def _lib():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventCreate.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.restype = ctypes.c_int
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.restype = ctypes.c_int
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.restype = ctypes.c_int
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventRecord.restype = ctypes.c_int
        _hip = h
    return _hip


class HipEvent:
    def __init__(self):
        self.handle = ctypes.c_void_p()
        rc = _lib().hipEventCreate(ctypes.byref(self.handle))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")

    @property
    def ptr(self) -> int:
        return self.handle.value

    def record(self, stream: int) -> None:
        rc = _lib().hipEventRecord(self.handle, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def synchronize(self) -> None:
        rc = _lib().hipEventSynchronize(self.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = _lib().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            if self.handle and _hip is not None:
                _hip.hipEventDestroy(self.handle)
        except Exception:
            pass
