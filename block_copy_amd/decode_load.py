"""ctypes binding of libkvload.so (measurement only): the synthetic bf16 GEMV
decode loop that the interference benchmark runs next to copy bursts (and an
ALU-only stand-in for it), the scattered read-only and write-only passes
that bound the D2D copy, and an empty kernel for launch floors."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvload.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"libkvload.so not built ({LIB_PATH})")
lib = ctypes.CDLL(LIB_PATH)
lib.kvload_gemv_bf16.restype = ctypes.c_int
lib.kvload_gemv_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p]
lib.kvload_chain_bf16.restype = ctypes.c_int
lib.kvload_chain_bf16.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_void_p),
                                  ctypes.c_int, ctypes.c_void_p]

lib.kvload_alu_chain.restype = ctypes.c_int
lib.kvload_alu_chain.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
lib.kvload_empty.restype = ctypes.c_int
lib.kvload_empty.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]

for _f in (lib.kvload_gather_read, lib.kvload_scatter_write):
    _f.restype = ctypes.c_int
lib.kvload_gather_read.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
lib.kvload_scatter_write.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32,
                                     ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]


def _stream(s):
    if s is None:
        return None
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def gemv(W, x, y, stream=None) -> None:
    """y = W @ x for bf16 torch tensors W [rows, cols], x [cols], y [rows] (on the GPU)."""
    rows, cols = W.shape
    if x.numel() != cols or y.numel() != rows or not (W.is_contiguous() and x.is_contiguous()
                                                      and y.is_contiguous()):
        raise ValueError("shape or layout mismatch")
    rc = lib.kvload_gemv_bf16(W.data_ptr(), x.data_ptr(), y.data_ptr(), rows, cols, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"kvload_gemv_bf16 failed: hipError {rc}")


class Chain:
    """A decode step: products W[i] @ acts[i] -> acts[i+1] for i in order."""

    def __init__(self, weights, acts):
        n = len(weights)
        if len(acts) != n + 1:
            raise ValueError("need len(weights) + 1 activation buffers")
        for i, W in enumerate(weights):
            r, c = W.shape
            if acts[i].numel() != c or acts[i + 1].numel() != r:
                raise ValueError(f"activation size mismatch at product {i}")
        self.n = n
        self._keep = (weights, acts)
        self.Ws = (ctypes.c_void_p * n)(*[W.data_ptr() for W in weights])
        self.rows = (ctypes.c_int * n)(*[W.shape[0] for W in weights])
        self.cols = (ctypes.c_int * n)(*[W.shape[1] for W in weights])
        self.acts = (ctypes.c_void_p * (n + 1))(*[a.data_ptr() for a in acts])

    def run(self, stream=None) -> None:
        rc = lib.kvload_chain_bf16(self.Ws, self.rows, self.cols, self.acts, self.n, _stream(stream))
        if rc != 0:
            raise RuntimeError(f"kvload_chain_bf16 failed: hipError {rc}")


class AluChain:
    """The ALU-only stand-in for a decode step: n kernels of `grid`
    workgroups, each thread running `iters` dependent FMAs, one store per
    workgroup at the end (`out`: a GPU float tensor of at least 1,024)."""

    def __init__(self, out, n=36, grid=1024, iters=4096):
        if out.numel() < 1024 or not out.is_cuda or out.element_size() != 4:
            raise ValueError("out must be a float32 GPU tensor of at least 1,024 elements")
        self.out, self.n, self.grid, self.iters = out, int(n), int(grid), int(iters)

    def run(self, stream=None) -> None:
        rc = lib.kvload_alu_chain(self.out.data_ptr(), self.n, self.grid, self.iters, _stream(stream))
        if rc != 0:
            raise RuntimeError(f"kvload_alu_chain failed: hipError {rc}")


def empty(grid, stream=None, start=None, stop=None) -> None:
    """One empty kernel of `grid` workgroups (its events give the launch floor)."""
    rc = lib.kvload_empty(int(grid), _stream(stream), start, stop)
    if rc != 0:
        raise RuntimeError(f"kvload_empty failed: hipError {rc}")


def _blocks(addrs, block_bytes):
    if addrs.dtype.itemsize != 8 or not addrs.is_cuda or not addrs.is_contiguous():
        raise ValueError("addrs must be a contiguous 64-bit tensor on the GPU")
    n = addrs.numel()
    if n == 0 or n > 1 << 30 or block_bytes <= 0 or block_bytes % 16 or block_bytes > 16384:
        raise ValueError("need 0 < n <= 2**30 and a block size that is a multiple of 16, <= 16 KiB")
    return n


def gather_read(addrs, block_bytes, sink, stream=None, start=None, stop=None) -> None:
    """Read the blocks at the device addresses in `addrs` (int64 tensor on the
    GPU); `sink` is a GPU tensor of at least 256 bytes, written only if the
    folded data equals a fixed value.  start/stop: raw hipEvent_t handles."""
    n = _blocks(addrs, block_bytes)
    if sink.numel() * sink.element_size() < 256 or not sink.is_cuda:
        raise ValueError("sink must be a GPU tensor of at least 256 bytes")
    rc = lib.kvload_gather_read(addrs.data_ptr(), n, block_bytes, 0x9E3779B9, sink.data_ptr(),
                                _stream(stream), start, stop)
    if rc != 0:
        raise RuntimeError(f"kvload_gather_read failed: hipError {rc}")


def scatter_write(addrs, block_bytes, pattern, stream=None, start=None, stop=None) -> None:
    """Fill the blocks at the device addresses in `addrs` with a 32-bit pattern."""
    n = _blocks(addrs, block_bytes)
    rc = lib.kvload_scatter_write(addrs.data_ptr(), n, block_bytes, pattern & 0xFFFFFFFF,
                                  _stream(stream), start, stop)
    if rc != 0:
        raise RuntimeError(f"kvload_scatter_write failed: hipError {rc}")
