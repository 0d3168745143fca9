"""Minimal ctypes access to the HIP runtime for timing and baselines.

Used by bench.py and the tests for events on a given stream and for the
baselines that use the runtime's own copies (contiguous ceilings, one
hipMemcpyAsync per fragment, one hipMemcpyBatchAsync per list; kernel
traces show the runtime carrying the contiguous and per-fragment copies
out as its own blit kernel).  In a process that has imported torch,
the HIP runtime already loaded is torch's own copy, and this module (like
libkvcopy.so) binds to it.
"""
from __future__ import annotations

import ctypes
import ctypes.util
import os
import sys

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
hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
hip.hipFree.argtypes = [ctypes.c_void_p]
hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
hip.hipHostFree.argtypes = [ctypes.c_void_p]
hip.hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
hip.hipRuntimeGetVersion.argtypes = [ctypes.POINTER(ctypes.c_int)]
hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]


class _MemLocation(ctypes.Structure):
    """hipMemLocation."""
    _fields_ = [("type", ctypes.c_int), ("id", ctypes.c_int)]


class _MemcpyAttributes(ctypes.Structure):
    """hipMemcpyAttributes."""
    _fields_ = [("srcAccessOrder", ctypes.c_int), ("srcLocHint", _MemLocation),
                ("dstLocHint", _MemLocation), ("flags", ctypes.c_uint)]


_SRC_ACCESS_ORDER_STREAM = 1                    # hipMemcpySrcAccessOrderStream
_LOC_DEVICE, _LOC_HOST = 1, 2                    # hipMemLocationTypeDevice / Host
_u64p = ctypes.POINTER(ctypes.c_uint64)
_has_batch = hasattr(hip, "hipMemcpyBatchAsync")
if _has_batch:
    hip.hipMemcpyBatchAsync.argtypes = [_u64p, _u64p, _u64p, ctypes.c_size_t,
                                        ctypes.POINTER(_MemcpyAttributes), _u64p, ctypes.c_size_t,
                                        _u64p, ctypes.c_void_p]
    hip.hipMemcpyBatchAsync.restype = ctypes.c_int
for _f in ("hipEventCreate", "hipEventRecord", "hipEventSynchronize", "hipEventElapsedTime",
           "hipEventDestroy", "hipMemcpyAsync", "hipStreamSynchronize", "hipDeviceSynchronize",
           "hipExtStreamCreateWithCUMask", "hipStreamDestroy", "hipMalloc", "hipFree",
           "hipHostMalloc", "hipHostFree", "hipMemset", "hipStreamCreate", "hipRuntimeGetVersion",
           "hipEventCreateWithFlags", "hipStreamWaitEvent"):
    getattr(hip, _f).restype = ctypes.c_int


def check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with hipError {rc}")


class Event:
    def __init__(self, timing: bool = True):
        h = ctypes.c_void_p()
        if timing:
            check(hip.hipEventCreate(ctypes.byref(h)), "hipEventCreate")
        else:   # hipEventDisableTiming: an ordering marker only
            check(hip.hipEventCreateWithFlags(ctypes.byref(h), 2), "hipEventCreateWithFlags")
        self.h = h.value

    def record(self, stream) -> None:
        check(hip.hipEventRecord(self.h, _s(stream)), "hipEventRecord")

    def elapsed_ms(self, end: "Event") -> float:
        check(hip.hipEventSynchronize(end.h), "hipEventSynchronize")
        ms = ctypes.c_float()
        check(hip.hipEventElapsedTime(ctypes.byref(ms), self.h, end.h), "hipEventElapsedTime")
        return float(ms.value)

    def destroy(self) -> None:
        if self.h:
            h, self.h = self.h, None
            check(hip.hipEventDestroy(h), "hipEventDestroy")

    def __del__(self, _finalizing=sys.is_finalizing):
        # No HIP call from a finaliser that runs while the interpreter shuts
        # down: by then the runtime (or a profiler wrapped around it) may be
        # tearing itself down.  The process's exit releases the event.
        # (sys.is_finalizing is bound as a default: module globals may
        # already be cleared when a late finaliser runs)
        if _finalizing():
            return
        try:
            self.destroy()
        except Exception:
            pass


def _s(stream):
    if stream is None:
        return None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def memcpy_async(dst: int, src: int, nbytes: int, kind: int, stream) -> None:
    check(hip.hipMemcpyAsync(dst, src, nbytes, kind, _s(stream)), "hipMemcpyAsync")


def memcpy_batch_async(dsts, srcs, sizes, stream, src_host: bool, dst_host: bool,
                       with_attrs: bool = True) -> int:
    """One hipMemcpyBatchAsync call for the whole list (the runtime's batched
    DMA path), in stream order; dsts/srcs/sizes are uint64 NumPy arrays of
    equal length.  with_attrs=False passes no copy attributes (the runtime's
    header marks them unsupported).  Returns the hipError_t (0 on success);
    raises if the runtime does not export the call."""
    import numpy as np
    if not _has_batch:
        raise RuntimeError("hipMemcpyBatchAsync is not exported by this HIP runtime")
    d = np.ascontiguousarray(dsts, dtype=np.uint64)
    s = np.ascontiguousarray(srcs, dtype=np.uint64)
    z = np.ascontiguousarray(sizes, dtype=np.uint64)
    if not (len(d) == len(s) == len(z)):
        raise ValueError("dsts, srcs and sizes must have the same length")
    attrs = _MemcpyAttributes(_SRC_ACCESS_ORDER_STREAM,
                              _MemLocation(_LOC_HOST if src_host else _LOC_DEVICE, 0),
                              _MemLocation(_LOC_HOST if dst_host else _LOC_DEVICE, 0), 0)
    idx = np.zeros(1, np.uint64)
    fail = np.zeros(1, np.uint64)
    p = lambda a: a.ctypes.data_as(_u64p)  # noqa: E731
    if not with_attrs:
        return int(hip.hipMemcpyBatchAsync(p(d), p(s), p(z), len(d), None, None, 0, p(fail),
                                           _s(stream)))
    return int(hip.hipMemcpyBatchAsync(p(d), p(s), p(z), len(d), ctypes.byref(attrs), p(idx), 1,
                                       p(fail), _s(stream)))


def stream_sync(stream) -> None:
    check(hip.hipStreamSynchronize(_s(stream)), "hipStreamSynchronize")


def stream_wait(stream, event: "Event") -> None:
    """Work queued on `stream` after this waits for `event` (hipStreamWaitEvent)."""
    check(hip.hipStreamWaitEvent(_s(stream), event.h, 0), "hipStreamWaitEvent")


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


class QueueStreams:
    """n streams with a hardware queue each, for copies that must overlap.

    HIP multiplexes its streams onto a few hardware queues (GPU_MAX_HW_QUEUES,
    4 by default), and two streams that share one run their kernels one
    after the other.  Measured on MI355X with the bidirectional 16,384 x 4 KiB
    burst on two torch streams: in processes that created six streams before
    using any, the first two ran the directions back to back (55 GB/s) every
    time, another pair ran at 63-64 GB/s and the others at 85-88; with only
    the two streams, 3 processes in 8 ran at 75-80 GB/s.  A CU mask is a
    property of the hardware queue, so a stream created with one gets a
    queue of its own; with every CU in the mask it runs like any other
    stream (default priority).  torch.cuda.ExternalStream wraps them.

    `cus` (optional): one iterable of CU mask bits per stream instead of
    every CU.  Mask bit i is a CU of XCD i % 8, and a mask that leaves an
    XCD without CUs is refused."""

    def __init__(self, n: int, total_cus: int, cus=None):
        import torch
        if cus is not None and len(cus) != n:
            raise ValueError("cus must give one CU set per stream")
        sets = cus if cus is not None else [range(total_cus)] * n
        self._masked = [CUMaskStream(c, total_cus) for c in sets]
        self.streams = [torch.cuda.ExternalStream(m.cuda_stream) for m in self._masked]

    def destroy(self):
        for m in self._masked:
            m.destroy()
        self._masked, self.streams = [], []


def runtime_version() -> int:
    v = ctypes.c_int(0)
    check(hip.hipRuntimeGetVersion(ctypes.byref(v)), "hipRuntimeGetVersion")
    return int(v.value)


def has_memcpy_batch() -> bool:
    return _has_batch


def device_alloc(nbytes: int) -> int:
    p = ctypes.c_void_p()
    check(hip.hipMalloc(ctypes.byref(p), nbytes), "hipMalloc")
    return int(p.value)


def device_free(ptr: int) -> None:
    check(hip.hipFree(ctypes.c_void_p(ptr)), "hipFree")


def host_alloc_mapped(nbytes: int) -> int:
    """Pinned host memory, mapped and portable (device address == host address)."""
    p = ctypes.c_void_p()
    check(hip.hipHostMalloc(ctypes.byref(p), nbytes, 0x2 | 0x1), "hipHostMalloc")
    return int(p.value)


def host_free(ptr: int) -> None:
    check(hip.hipHostFree(ctypes.c_void_p(ptr)), "hipHostFree")


def memset(ptr: int, value: int, nbytes: int) -> None:
    check(hip.hipMemset(ctypes.c_void_p(ptr), value, nbytes), "hipMemset")


def stream_create() -> int:
    h = ctypes.c_void_p()
    check(hip.hipStreamCreate(ctypes.byref(h)), "hipStreamCreate")
    return int(h.value)
