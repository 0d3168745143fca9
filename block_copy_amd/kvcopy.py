"""ctypes binding of libkvcopy.so (include/kvcopy.h): argument marshalling only.

Every step of the copy runs inside the library (host planner + gfx950
kernel).  This module never computes a result itself and has no fallback:
if the library is missing or cannot be loaded, importing it raises.

Descriptor arrays may be NumPy arrays, CPU torch tensors or sequences of
ints; they are passed as contiguous uint64 buffers.  Streams are HIP stream
handles as integers (``torch.cuda.current_stream().cuda_stream`` on ROCm) or
None for the null stream.
"""
from __future__ import annotations

import ctypes
import os
import sys
from dataclasses import dataclass

import numpy as np

H2D, D2H, D2D = 0, 1, 2
OK, EINVAL, EALIGN, EOVERLAP, ENOMEM, EHIP = 0, -1, -2, -3, -4, -5
WGS_ALL, WGS_AUTO = 0, -1
CHUNK_DEFAULT = 16384
CHUNK_MAX = 1 << 20
F_VALIDATE, F_NO_COALESCE, F_DESC_UPLOAD = 0x1, 0x2, 0x8
F_PIPELINE, F_PER_CHUNK, F_DYNAMIC = 0x10, 0x20, 0x40
F_STORE_SC1, F_STORE_NT, F_DST_ORDER, F_TAIL_BOUNDED = 0x80, 0x100, 0x200, 0x400
F_WG_PER_CHUNK = 0x800
OPTS_V1_SIZE = 32

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvcopy.so")

# Every symbol include/kvcopy.h declares.
EXPORTS = ("kvcopy_coalesce", "kvcopy_plan", "kvcopy_plan_free", "kvcopy_batch",
           "kvcopy_batch_ex", "kvcopy_strerror", "kvcopy_last_hip_error",
           "kvcopy_host_alloc_mapped", "kvcopy_host_free", "kvcopy_job_create",
           "kvcopy_job_poll", "kvcopy_job_wait", "kvcopy_job_destroy",
           "kvcopy_device_workspace_bytes", "kvcopy_batch_device", "kvcopy_autotune",
           "kvcopy_batch_pair", "kvcopy_batch_device_noalloc")
DEVICE_BAD_ALIGN, DEVICE_TOO_MANY_CHUNKS = 1, 2
NOALLOC_MAX_N = 131072


class KvcopyError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = f"{where}: {kvcopy_strerror(code)} ({code})"
        if code == EHIP:
            msg += f", hipError {kvcopy_last_hip_error()}"
        super().__init__(msg)


class _Plan(ctypes.Structure):
    _fields_ = [("n_in", ctypes.c_uint64), ("n_merged", ctypes.c_uint64),
                ("n_chunks", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64),
                ("chunk_bytes", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("src", ctypes.POINTER(ctypes.c_uint64)), ("dst", ctypes.POINTER(ctypes.c_uint64)),
                ("size", ctypes.POINTER(ctypes.c_uint64)),
                ("chunk_begin", ctypes.POINTER(ctypes.c_uint64))]


class Opts(ctypes.Structure):
    """kvcopy_opts_t."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("chunk_bytes", ctypes.c_uint32),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("kernel_begin", ctypes.c_void_p), ("kernel_end", ctypes.c_void_p),
                ("duty_on_ns", ctypes.c_uint32), ("duty_period_ns", ctypes.c_uint32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libkvcopy.so not built ({LIB_PATH}); run "
                          "`python -m block_copy_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.kvcopy_coalesce.restype = ctypes.c_int
    lib.kvcopy_coalesce.argtypes = [u64p, u64p, u64p, ctypes.c_uint64, u64p, u64p, u64p, u64p]
    lib.kvcopy_plan.restype = ctypes.c_int
    lib.kvcopy_plan.argtypes = [u64p, u64p, u64p, ctypes.c_uint64, ctypes.c_uint32,
                                ctypes.POINTER(_Plan)]
    lib.kvcopy_plan_free.restype = None
    lib.kvcopy_plan_free.argtypes = [ctypes.POINTER(_Plan)]
    lib.kvcopy_batch.restype = ctypes.c_int
    lib.kvcopy_batch.argtypes = [u64p, u64p, u64p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    lib.kvcopy_batch_ex.restype = ctypes.c_int
    lib.kvcopy_batch_ex.argtypes = [u64p, u64p, u64p, ctypes.c_uint64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(Opts)]
    lib.kvcopy_batch_pair.restype = ctypes.c_int
    lib.kvcopy_batch_pair.argtypes = [u64p, u64p, u64p, ctypes.c_uint64, u64p, u64p, u64p,
                                      ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32,
                                      ctypes.c_void_p]
    lib.kvcopy_strerror.restype = ctypes.c_char_p
    lib.kvcopy_strerror.argtypes = [ctypes.c_int]
    lib.kvcopy_last_hip_error.restype = ctypes.c_int
    lib.kvcopy_last_hip_error.argtypes = []
    lib.kvcopy_host_alloc_mapped.restype = ctypes.c_int
    lib.kvcopy_host_alloc_mapped.argtypes = [ctypes.c_uint64, ctypes.POINTER(ctypes.c_void_p)]
    lib.kvcopy_host_free.restype = ctypes.c_int
    lib.kvcopy_host_free.argtypes = [ctypes.c_void_p]
    lib.kvcopy_job_create.restype = ctypes.c_int
    lib.kvcopy_job_create.argtypes = [u64p, u64p, u64p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.POINTER(ctypes.c_void_p)]
    lib.kvcopy_job_poll.restype = ctypes.c_int
    lib.kvcopy_job_poll.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    lib.kvcopy_job_wait.restype = ctypes.c_int
    lib.kvcopy_job_wait.argtypes = [ctypes.c_void_p]
    lib.kvcopy_job_destroy.restype = None
    lib.kvcopy_job_destroy.argtypes = [ctypes.c_void_p]
    lib.kvcopy_autotune.restype = ctypes.c_int
    lib.kvcopy_autotune.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]
    lib.kvcopy_device_workspace_bytes.restype = ctypes.c_uint64
    lib.kvcopy_device_workspace_bytes.argtypes = [ctypes.c_uint64]
    lib.kvcopy_batch_device.restype = ctypes.c_int
    lib.kvcopy_batch_device.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.kvcopy_batch_device_noalloc.restype = ctypes.c_int
    lib.kvcopy_batch_device_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p,
                                                ctypes.c_void_p]
    return lib


lib = _load()


def _u64(a):
    """(keep-alive array, uint64* pointer) for an int sequence / ndarray / CPU tensor."""
    if a is None:
        return None, None
    if hasattr(a, "numpy") and hasattr(a, "device"):       # torch tensor
        if a.device.type != "cpu":
            raise ValueError("descriptor arrays must be host (CPU) arrays")
        a = a.numpy()
    arr = np.asarray(a)
    if arr.dtype != np.uint64:
        arr = arr.astype(np.uint64)
    arr = np.ascontiguousarray(arr)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))


def _n(*arrays):
    lens = {len(x) for x in arrays if x is not None}
    if len(lens) > 1:
        raise ValueError("src, dst and sizes must have the same length")
    return lens.pop() if lens else 0


def kvcopy_strerror(code: int) -> str:
    return lib.kvcopy_strerror(int(code)).decode()


def kvcopy_last_hip_error() -> int:
    return int(lib.kvcopy_last_hip_error())


def kvcopy_coalesce(src, dst, sizes, raw: bool = False):
    """Merged (src, dst, sizes) uint64 arrays.  raw=True returns (code, arrays)."""
    s, sp = _u64(src)
    d, dp = _u64(dst)
    z, zp = _u64(sizes)
    n = _n(s, d, z)
    os_ = np.empty(n, np.uint64)
    od = np.empty(n, np.uint64)
    oz = np.empty(n, np.uint64)
    m = ctypes.c_uint64(0)
    p = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))  # noqa: E731
    rc = lib.kvcopy_coalesce(sp, dp, zp, n, p(os_), p(od), p(oz), ctypes.byref(m))
    out = (os_[:m.value], od[:m.value], oz[:m.value])
    if raw:
        return rc, out
    if rc != OK:
        raise KvcopyError(rc, "kvcopy_coalesce")
    return out


@dataclass
class Plan:
    n_in: int
    n_merged: int
    n_chunks: int
    total_bytes: int
    chunk_bytes: int
    src: np.ndarray
    dst: np.ndarray
    size: np.ndarray
    chunk_begin: np.ndarray


def kvcopy_plan(src, dst, sizes, chunk_bytes: int = 0) -> Plan:
    """Validated, coalesced and chunked plan (copied out of the library)."""
    s, sp = _u64(src)
    d, dp = _u64(dst)
    z, zp = _u64(sizes)
    n = _n(s, d, z)
    plan = _Plan()
    rc = lib.kvcopy_plan(sp, dp, zp, n, int(chunk_bytes), ctypes.byref(plan))
    if rc != OK:
        raise KvcopyError(rc, "kvcopy_plan")
    try:
        m = plan.n_merged

        def grab(ptr, k):
            return np.ctypeslib.as_array(ptr, shape=(k,)).copy() if k else np.zeros(0, np.uint64)
        return Plan(plan.n_in, m, plan.n_chunks, plan.total_bytes, plan.chunk_bytes,
                    grab(plan.src, m), grab(plan.dst, m), grab(plan.size, m),
                    grab(plan.chunk_begin, m + 1))
    finally:
        lib.kvcopy_plan_free(ctypes.byref(plan))


def kvcopy_batch(src_addrs, dst_addrs, sizes, dir: int, max_wgs: int = WGS_ALL,
                 stream=None, *, chunk_bytes: int = 0, flags: int = 0,
                 kernel_begin=None, kernel_end=None, duty_on_ns: int = 0,
                 duty_period_ns: int = 0, opts_size: int = 0, check: bool = True) -> int:
    """Enqueue the batch on `stream` (see include/kvcopy.h).

    With any option given, calls kvcopy_batch_ex.  kernel_begin/kernel_end
    are raw hipEvent_t handles (ints).  opts_size overrides struct_size
    (say OPTS_V1_SIZE).  Raises KvcopyError on failure unless check=False,
    in which case the status code is returned.
    """
    s, sp = _u64(src_addrs)
    d, dp = _u64(dst_addrs)
    z, zp = _u64(sizes)
    n = _n(s, d, z)
    st = ctypes.c_void_p(int(stream) if stream else 0)
    if chunk_bytes or flags or kernel_begin or kernel_end or duty_period_ns or opts_size:
        o = Opts(int(opts_size) or ctypes.sizeof(Opts), int(chunk_bytes), int(flags), 0,
                 ctypes.c_void_p(int(kernel_begin) if kernel_begin else 0),
                 ctypes.c_void_p(int(kernel_end) if kernel_end else 0),
                 int(duty_on_ns), int(duty_period_ns))
        rc = lib.kvcopy_batch_ex(sp, dp, zp, n, int(dir), int(max_wgs), st, ctypes.byref(o))
    else:
        rc = lib.kvcopy_batch(sp, dp, zp, n, int(dir), int(max_wgs), st)
    if check and rc != OK:
        raise KvcopyError(rc, "kvcopy_batch")
    return rc


def kvcopy_batch_pair(src_a, dst_a, sizes_a, src_b, dst_b, sizes_b, max_wgs: int = WGS_ALL,
                      stream=None, *, flags: int = 0, check: bool = True) -> int:
    """Two descriptor lists in one launch on `stream` (see include/kvcopy.h)."""
    sa, sap = _u64(src_a)
    da, dap = _u64(dst_a)
    za, zap = _u64(sizes_a)
    sb, sbp = _u64(src_b)
    db, dbp = _u64(dst_b)
    zb, zbp = _u64(sizes_b)
    na, nb = _n(sa, da, za), _n(sb, db, zb)
    st = ctypes.c_void_p(int(stream) if stream else 0)
    rc = lib.kvcopy_batch_pair(sap, dap, zap, na, sbp, dbp, zbp, nb, int(max_wgs), int(flags), st)
    if check and rc != OK:
        raise KvcopyError(rc, "kvcopy_batch_pair")
    return rc


def kvcopy_host_alloc_mapped(nbytes: int) -> int:
    """Mapped pinned host memory; returns its address (same on host and GPU)."""
    p = ctypes.c_void_p(0)
    rc = lib.kvcopy_host_alloc_mapped(int(nbytes), ctypes.byref(p))
    if rc != OK:
        raise KvcopyError(rc, "kvcopy_host_alloc_mapped")
    return int(p.value)


def kvcopy_host_free(ptr: int) -> None:
    rc = lib.kvcopy_host_free(ctypes.c_void_p(int(ptr) if ptr else 0))
    if rc != OK:
        raise KvcopyError(rc, "kvcopy_host_free")


class HostBuffer:
    """Mapped pinned host memory viewed as a NumPy uint8 array."""

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self.ptr = kvcopy_host_alloc_mapped(self.nbytes)
        self.array = np.ctypeslib.as_array((ctypes.c_uint8 * self.nbytes).from_address(self.ptr))

    def free(self):
        if self.ptr:
            self.array = None
            kvcopy_host_free(self.ptr)
            self.ptr = 0

    def __del__(self, _finalizing=sys.is_finalizing):
        # Free explicitly (free()); a finaliser that runs during interpreter
        # shutdown makes no HIP call and leaves the memory to the process's
        # exit.
        # (sys.is_finalizing is bound as a default: module globals may
        # already be cleared when a late finaliser runs)
        if _finalizing():
            return
        try:
            self.free()
        except Exception:
            pass


def kvcopy_job_create(src_addrs, dst_addrs, sizes, dir: int, max_wgs: int = WGS_ALL,
                      piece_descs: int = 0, stream=None) -> int:
    """A paced job (see include/kvcopy.h); returns its handle."""
    s, sp = _u64(src_addrs)
    d, dp = _u64(dst_addrs)
    z, zp = _u64(sizes)
    n = _n(s, d, z)
    h = ctypes.c_void_p(0)
    st = ctypes.c_void_p(int(stream) if stream else 0)
    rc = lib.kvcopy_job_create(sp, dp, zp, n, int(dir), int(max_wgs), int(piece_descs), st,
                               ctypes.byref(h))
    if rc != OK:
        raise KvcopyError(rc, "kvcopy_job_create")
    return int(h.value)


def kvcopy_job_poll(job: int) -> bool:
    """Submits the next piece if the previous one completed; True once all completed."""
    done = ctypes.c_int(0)
    rc = lib.kvcopy_job_poll(ctypes.c_void_p(job), ctypes.byref(done))
    if rc != OK:
        raise KvcopyError(rc, "kvcopy_job_poll")
    return bool(done.value)


def kvcopy_job_wait(job: int) -> None:
    rc = lib.kvcopy_job_wait(ctypes.c_void_p(job))
    if rc != OK:
        raise KvcopyError(rc, "kvcopy_job_wait")


def kvcopy_job_destroy(job: int) -> None:
    lib.kvcopy_job_destroy(ctypes.c_void_p(job))


def kvcopy_device_workspace_bytes(max_n: int) -> int:
    return int(lib.kvcopy_device_workspace_bytes(int(max_n)))


def kvcopy_batch_device(d_src: int, d_dst: int, d_sizes: int, d_n: int, max_n: int, dir: int,
                        max_wgs: int, workspace: int, stream=None, chunk_bytes: int = 0,
                        check: bool = True) -> int:
    """Device-resident batch (see include/kvcopy.h).  All pointers are device
    addresses (ints), e.g. torch tensors' data_ptr()."""
    st = ctypes.c_void_p(int(stream) if stream else 0)
    p = lambda x: ctypes.c_void_p(int(x) if x else 0)  # noqa: E731
    rc = lib.kvcopy_batch_device(p(d_src), p(d_dst), p(d_sizes), p(d_n), int(max_n), int(dir),
                                 int(max_wgs), int(chunk_bytes), p(workspace), st)
    if check and rc != OK:
        raise KvcopyError(rc, "kvcopy_batch_device")
    return rc


def kvcopy_batch_device_noalloc(d_src: int, d_dst: int, d_sizes: int, d_n: int, max_n: int,
                                dir: int, max_wgs: int, d_status: int = 0, stream=None,
                                chunk_bytes: int = 0, check: bool = True) -> int:
    """kvcopy_batch_device with the library's own workspace (see
    include/kvcopy.h): no allocation; max_n <= NOALLOC_MAX_N; d_status is
    an optional device address that receives the status word."""
    st = ctypes.c_void_p(int(stream) if stream else 0)
    p = lambda x: ctypes.c_void_p(int(x) if x else 0)  # noqa: E731
    rc = lib.kvcopy_batch_device_noalloc(p(d_src), p(d_dst), p(d_sizes), p(d_n), int(max_n),
                                         int(dir), int(max_wgs), int(chunk_bytes), p(d_status), st)
    if check and rc != OK:
        raise KvcopyError(rc, "kvcopy_batch_device_noalloc")
    return rc


AUTOTUNE_CAPS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 0)


def kvcopy_autotune(dir: int, s0=None, s1=None):
    """Run the startup probe for `dir` on the current device (see include/kvcopy.h).
    Returns (chosen cap, {cap: GB/s})."""
    w = ctypes.c_int(0)
    rates = (ctypes.c_double * len(AUTOTUNE_CAPS))()
    p = lambda x: ctypes.c_void_p(int(x) if x else 0)  # noqa: E731
    rc = lib.kvcopy_autotune(int(dir), p(s0), p(s1), ctypes.byref(w), rates)
    if rc != OK:
        raise KvcopyError(rc, "kvcopy_autotune")
    return int(w.value), {c: rates[i] / 1e9 for i, c in enumerate(AUTOTUNE_CAPS)}
