"""The pins catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/oracle.c (on the CPU only),
compiles it with gcc, and checks that the brute-force and fixture pins of
test_oracle.py reject it.  The unmodified source must pass the same checks.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
GOLDEN = os.path.join(ROOT, "tests", "golden")

MUTANTS = {
    "none": [],
    "drop_last_word": [("memcpy(d, s, size[i]);", "memcpy(d, s, size[i] - 8);")],
    "drop_last_descriptor": [("i < n; ++i", "i + 1 < n; ++i")],
    "swapped_operands": [("memcpy(d, s, size[i]);", "memcpy((uint8_t *)s, d, size[i]);")],
    "offset_off_by_word": [("return r->img + (addr - r->base);", "return r->img + (addr - r->base) + (addr > r->base ? 8 : 0);")],
    "size_of_wrong_descriptor": [("memcpy(d, s, size[i]);", "memcpy(d, s, size[i + 1 < n ? i + 1 : i] < size[i] ? size[i + 1 < n ? i + 1 : i] : size[i]);")],
    "dst_written_in_source_image": [("uint8_t *d = oracle_locate(dst_arenas, n_dst, dst[i], size[i]);",
                                     "uint8_t *d = oracle_locate(dst_arenas, n_dst, dst[i], size[i]); if (d) d = (uint8_t *)s;")],
    "skip_second_descriptor": [("if (size[i] == 0)", "if (size[i] == 0 || i == 1)")],
}


class _Arena(ctypes.Structure):
    _fields_ = [("base", ctypes.c_uint64), ("len", ctypes.c_uint64), ("img", ctypes.c_void_p)]


def _build(tmp_path, name, edits):
    src = SRC
    for old, new in edits:
        assert old in src, (name, old)
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-shared", "-fPIC", str(c), "-o", str(so)], check=True)
    lib = ctypes.CDLL(str(so))
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.oracle_copy.restype = ctypes.c_int64
    lib.oracle_copy.argtypes = [u64p, u64p, u64p, ctypes.c_uint64, ctypes.POINTER(_Arena),
                                ctypes.c_int, ctypes.POINTER(_Arena), ctypes.c_int, u64p]
    return lib


def _call(lib, descs, src_arenas, dst_arenas):
    a = np.ascontiguousarray(np.array(descs, dtype=np.uint64).reshape(-1, 3).T)
    p = [np.ascontiguousarray(a[k]) for k in range(3)]
    u64p = ctypes.POINTER(ctypes.c_uint64)
    sa = (_Arena * len(src_arenas))(*[_Arena(b, len(i), i.ctypes.data) for b, i in src_arenas])
    dsts = [(b, i.copy()) for b, i in dst_arenas]
    da = (_Arena * len(dsts))(*[_Arena(b, len(i), i.ctypes.data) for b, i in dsts])
    moved = ctypes.c_uint64(0)
    rc = lib.oracle_copy(*(x.ctypes.data_as(u64p) for x in p), len(descs), sa, len(src_arenas),
                         da, len(dsts), ctypes.byref(moved))
    return rc, [i for _, i in dsts], moved.value


def _pins_pass(lib):
    """A compact version of the oracle's pins; returns False on the first failure."""
    for c in json.load(open(os.path.join(GOLDEN, "copy_cases.json")))["cases"]:
        src = [(a["base"], ((a["src_fill_base"] + np.arange(a["len"])) % 256).astype(np.uint8))
               for a in c["src_arenas"]]
        dst = [(a["base"], np.full(a["len"], a["dst_fill"], np.uint8)) for a in c["dst_arenas"]]
        rc, out, moved = _call(lib, c["descs"], src, dst)
        if rc != 0 or moved != c["bytes_moved"]:
            return False
        if [o.tobytes().hex() for o in out] != c["expect_hex_per_dst_arena"]:
            return False
    from test_oracle import brute_force
    rng = np.random.default_rng(3)
    S = (0x10000, rng.integers(0, 256, 128, dtype=np.uint8))
    D = (0x30000, np.full(128, 0xA5, np.uint8))
    for _ in range(300):
        k = int(rng.integers(1, 4))
        descs, used = [], np.zeros(128, bool)
        for _ in range(k):
            n = int(rng.choice([8, 16, 24, 40]))
            do = 8 * int(rng.integers(0, (128 - n) // 8 + 1))
            if used[do:do + n].any():
                continue
            used[do:do + n] = True
            descs.append((S[0] + 8 * int(rng.integers(0, (128 - n) // 8 + 1)), D[0] + do, n))
        rc, out, _ = _call(lib, descs, [S], [D])
        if rc != 0 or not np.array_equal(out[0], brute_force(descs, [S], [D])[0]):
            return False
    return True


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant(tmp_path, name):
    lib = _build(tmp_path, name, MUTANTS[name])
    if name == "none":
        assert _pins_pass(lib)
    else:
        assert not _pins_pass(lib), f"planted mistake '{name}' was not caught"
