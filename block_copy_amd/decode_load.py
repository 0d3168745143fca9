"""ctypes binding of libkvload.so: the synthetic bf16 GEMV decode loop that the
interference benchmark runs next to copy bursts (measurement only)."""
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
