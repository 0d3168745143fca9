"""The CPU oracle for the batched descriptor copy.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  It shares no code with the product
library (block_copy_amd/), and the product never imports it.

Parts:
  oracle.c  -- ``oracle_copy``: one memcpy per descriptor into host images of
               the arenas the batch touches (the definition of the result).
  plan.py   -- coalescing and chunking written out from their definitions.

Citations for each step are in the headers of those two files.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import plan  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build_lib() -> str:
    """Compile oracle.c with gcc -O3 into liboracle.so next to it."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O3", "-std=c11", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC",
                    _SRC, "-o", tmp], check=True)
    os.replace(tmp, _LIB)
    return _LIB


class _Arena(ctypes.Structure):
    _fields_ = [("base", ctypes.c_uint64), ("len", ctypes.c_uint64), ("img", ctypes.c_void_p)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_lib()
        lib = ctypes.CDLL(_LIB)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        lib.oracle_copy.restype = ctypes.c_int64
        lib.oracle_copy.argtypes = [u64p, u64p, u64p, ctypes.c_uint64,
                                    ctypes.POINTER(_Arena), ctypes.c_int,
                                    ctypes.POINTER(_Arena), ctypes.c_int, u64p]
        _lib = lib
    return _lib


def _u64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))


def _arenas(arenas, writable):
    arr = (_Arena * max(1, len(arenas)))()
    for i, (base, img) in enumerate(arenas):
        if img.dtype != np.uint8 or not img.flags["C_CONTIGUOUS"]:
            raise TypeError("arena images must be C-contiguous uint8 arrays")
        if writable and not img.flags["WRITEABLE"]:
            raise TypeError("destination images must be writable")
        arr[i].base = int(base)
        arr[i].len = img.nbytes
        arr[i].img = img.ctypes.data
    return arr


def copy(src, dst, size, src_arenas, dst_arenas):
    """Apply the batch to host images.

    ``src_arenas`` / ``dst_arenas``: lists of (base_address, uint8 ndarray).
    The destination arrays are modified in place.  Returns the bytes moved.
    Raises ValueError if a descriptor lies outside every arena.
    """
    lib = _load()
    s, sp = _u64(src)
    d, dp = _u64(dst)
    n, np_ = _u64(size)
    if not (len(s) == len(d) == len(n)):
        raise ValueError("src, dst and size must have the same length")
    sa = _arenas(src_arenas, False)
    da = _arenas(dst_arenas, True)
    moved = ctypes.c_uint64(0)
    rc = lib.oracle_copy(sp, dp, np_, len(n), sa, len(src_arenas), da, len(dst_arenas),
                         ctypes.byref(moved))
    if rc != 0:
        raise ValueError(f"descriptor {-rc - 1} lies outside every arena")
    return int(moved.value)
