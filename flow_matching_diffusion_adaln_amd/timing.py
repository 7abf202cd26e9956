"""HIP events through ctypes, for timing work on a given stream.

torch.cuda.Event only records on torch's current stream and hides its
handle; these are plain hipEvent_t handles from the HIP runtime that torch
itself has loaded, so they can be recorded by the library on any stream.
"""
from __future__ import annotations

import ctypes
import ctypes.util

_hip = None


def hip() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so", mode=ctypes.RTLD_GLOBAL)
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
    return _hip


def create(n: int):
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        rc = hip().hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        evs.append(e.value)
    return evs


def record(ev, stream_handle: int) -> None:
    rc = hip().hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream_handle))
    if rc != 0:
        raise RuntimeError(f"hipEventRecord failed ({rc})")


def elapsed_ms(a, b) -> float:
    hip().hipEventSynchronize(ctypes.c_void_p(b))
    ms = ctypes.c_float()
    rc = hip().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
    return ms.value


def destroy(evs) -> None:
    for e in evs:
        hip().hipEventDestroy(ctypes.c_void_p(e))
