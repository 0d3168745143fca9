"""Pins for the planning oracle (oracle/plan.py).

* Hand-derived fixtures under tests/golden/ for coalescing and chunking.
* Coalescing preserves the byte mapping: on random tiny inputs, the set of
  (destination byte <- source byte) pairs is identical before and after.
* Coalescing is maximal under its rule: no two consecutive outputs are
  adjacent in both source and destination, and no output has size zero.
* Chunking: closed-form count sum(ceil(s/C)), each chunk inside its range,
  at most C bytes, chunks tile each range exactly and in order.
"""
import json
import os

import numpy as np
import pytest

from oracle import plan as oplan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_coalesce():
    cases = json.load(open(os.path.join(GOLDEN, "coalesce_cases.json")))["cases"]
    assert len(cases) >= 10
    for c in cases:
        a = np.array(c["in"], dtype=np.uint64).reshape(-1, 3)
        s, d, n = oplan.coalesce(a[:, 0], a[:, 1], a[:, 2])
        assert [list(x) for x in zip(s, d, n)] == c["out"], c["name"]


def test_golden_chunks():
    cases = json.load(open(os.path.join(GOLDEN, "chunk_cases.json")))["cases"]
    for c in cases:
        C = c["chunk"]
        assert oplan.chunk_counts(c["sizes"], C) == c["counts"], c["name"]
        assert oplan.chunk_begin(c["sizes"], C) == c["begin"], c["name"]
        ch = oplan.chunks([0] * len(c["sizes"]), [0] * len(c["sizes"]), c["sizes"], C)
        if "chunk_bytes" in c:
            assert [x[2] for x in ch] == c["chunk_bytes"], c["name"]
        if "chunk_bytes_sum" in c:
            assert sum(x[2] for x in ch) == c["chunk_bytes_sum"], c["name"]


def _byte_map(src, dst, size):
    m = {}
    for s, d, n in zip(src, dst, size):
        for x in range(0, int(n), 8):       # 8 B granularity is enough: all offsets are 8 B multiples
            m[int(d) + x] = int(s) + x
    return m


def _random_descs(rng, n):
    """Tiny descriptor lists with many accidental adjacencies and zero sizes."""
    src, dst, size = [], [], []
    s, d = 0, 1 << 20
    for _ in range(n):
        sz = 8 * int(rng.integers(0, 4))
        if rng.random() < 0.5:       # continue in src
            pass
        else:
            s += 8 * int(rng.integers(-4, 8))
            s = max(s, 0)
        if rng.random() < 0.5:       # continue in dst
            pass
        else:
            d += 8 * int(rng.integers(1, 8))
        src.append(s); dst.append(d); size.append(sz)
        s += sz; d += sz
    return src, dst, size


def test_coalesce_preserves_byte_map_and_is_maximal():
    rng = np.random.default_rng(21)
    for trial in range(2000):
        src, dst, size = _random_descs(rng, int(rng.integers(0, 12)))
        cs, cd, cn = oplan.coalesce(src, dst, size)
        assert _byte_map(src, dst, size) == _byte_map(cs, cd, cn)
        assert sum(cn) == sum(size)
        assert all(n > 0 for n in cn)
        for i in range(len(cn) - 1):
            assert not (cs[i] + cn[i] == cs[i + 1] and cd[i] + cn[i] == cd[i + 1])
        assert len(cn) <= len([x for x in size if x])


@pytest.mark.parametrize("C", [16, 4096, 8192, 16384, 65536])
def test_chunk_partition(C):
    rng = np.random.default_rng(C)
    size = [8 * int(x) for x in rng.integers(1, 20000, 300)]
    src = [int(x) * 8 for x in rng.integers(0, 1 << 30, 300)]
    dst = [int(x) * 8 for x in rng.integers(0, 1 << 30, 300)]
    begin = oplan.chunk_begin(size, C)
    assert begin[-1] == sum(-(-s // C) for s in size)
    assert all(b < e for b, e in zip(begin, begin[1:]))
    ch = oplan.chunks(src, dst, size, C)
    assert len(ch) == begin[-1]
    for i in range(len(size)):
        mine = ch[begin[i]:begin[i + 1]]
        off = 0
        for s, d, n in mine:
            assert 0 < n <= C
            assert s == src[i] + off and d == dst[i] + off
            off += n
        assert off == size[i]
