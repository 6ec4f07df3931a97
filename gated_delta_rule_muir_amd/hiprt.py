"""Minimal ctypes access to the HIP runtime already loaded by torch (events only).

Used by the benchmark to hand raw hipEvent_t handles to
``muir_set_profile_events`` and read per-kernel durations back.
"""
from __future__ import annotations

import ctypes

_hip = None


def _rt():
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (loads the HIP runtime first; the same soname is reused)
        h = ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL)
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip = h
    return _hip


class EventPool:
    """`n` HIP events in a ctypes array suitable for muir_set_profile_events."""

    def __init__(self, n: int):
        rt = _rt()
        self.n = n
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            rc = rt.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.arr[i] = ev.value

    def elapsed_ms(self, i: int, j: int) -> float:
        rt = _rt()
        ms = ctypes.c_float()
        rt.hipEventSynchronize(ctypes.c_void_p(self.arr[j]))
        rc = rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.arr[i]), ctypes.c_void_p(self.arr[j]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self) -> None:
        rt = _rt()
        for i in range(self.n):
            if self.arr[i]:
                rt.hipEventDestroy(ctypes.c_void_p(self.arr[i]))
                self.arr[i] = None
