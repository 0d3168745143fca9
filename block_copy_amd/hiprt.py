"""Minimal ctypes access to the HIP runtime for timing and baselines.

Used by bench.py and the tests for events on a given stream and for the
plain hipMemcpyAsync baselines (contiguous ceilings, one copy per fragment).
"""
from __future__ import annotations

import ctypes
import ctypes.util
import os

_CANDIDATES = [os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "libamdhip64.so"),
               "libamdhip64.so"]

hip = None
for _p in _CANDIDATES:
    try:
        hip = ctypes.CDLL(_p)
        break
    except OSError:
        continue
if hip is None:
    raise ImportError("libamdhip64.so not found")

H2D_KIND, D2H_KIND, D2D_KIND = 1, 2, 3   # hipMemcpyHostToDevice, DeviceToHost, DeviceToDevice

hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                               ctypes.c_void_p]
hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
hip.hipDeviceSynchronize.argtypes = []
hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                             ctypes.POINTER(ctypes.c_uint32)]
hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
for _f in ("hipEventCreate", "hipEventRecord", "hipEventSynchronize", "hipEventElapsedTime",
           "hipEventDestroy", "hipMemcpyAsync", "hipStreamSynchronize", "hipDeviceSynchronize",
           "hipExtStreamCreateWithCUMask", "hipStreamDestroy"):
    getattr(hip, _f).restype = ctypes.c_int


def check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with hipError {rc}")


class Event:
    def __init__(self):
        h = ctypes.c_void_p()
        check(hip.hipEventCreate(ctypes.byref(h)), "hipEventCreate")
        self.h = h.value

    def record(self, stream) -> None:
        check(hip.hipEventRecord(self.h, _s(stream)), "hipEventRecord")

    def elapsed_ms(self, end: "Event") -> float:
        check(hip.hipEventSynchronize(end.h), "hipEventSynchronize")
        ms = ctypes.c_float()
        check(hip.hipEventElapsedTime(ctypes.byref(ms), self.h, end.h), "hipEventElapsedTime")
        return float(ms.value)

    def __del__(self):
        try:
            if self.h:
                hip.hipEventDestroy(self.h)
        except Exception:
            pass


def _s(stream):
    if stream is None:
        return None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def memcpy_async(dst: int, src: int, nbytes: int, kind: int, stream) -> None:
    check(hip.hipMemcpyAsync(dst, src, nbytes, kind, _s(stream)), "hipMemcpyAsync")


def stream_sync(stream) -> None:
    check(hip.hipStreamSynchronize(_s(stream)), "hipStreamSynchronize")


class CUMaskStream:
    """A stream whose kernels may run only on the given compute units
    (default priority).  `cus`: iterable of CU indices in [0, 256)."""

    def __init__(self, cus, total=256):
        words = (ctypes.c_uint32 * ((total + 31) // 32))()
        for c in cus:
            words[c // 32] |= 1 << (c % 32)
        h = ctypes.c_void_p()
        check(hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), len(words), words),
              "hipExtStreamCreateWithCUMask")
        self.cuda_stream = h.value

    def destroy(self):
        if self.cuda_stream:
            check(hip.hipStreamDestroy(self.cuda_stream), "hipStreamDestroy")
            self.cuda_stream = None
