"""GPU parity at the size limits and in the degenerate cases.

- One descriptor longer than 4 GiB (D2D, src = 8 mod 16), at the default
  and the largest chunk size: 64-bit offsets in the planner and the kernel.
  It is checked on sampled 64 KiB windows, including both ends and the guard
  bytes around the range. The oracle computes each window's expected bytes
  one by one from that window's source bytes.
- A million descriptors of 8..128 bytes in one call (H2D), also with 16-byte
  chunks (about 2.6 million chunks, so the staging ring grows several times).
  It is checked on the whole arenas.
- A chain of 16,384 adjacent 4 KiB descriptors that coalesces into a single
  64 MiB range, and the same list with coalescing switched off.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from test_gpu_parity import _check, _run, _say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_copy_amd import kvcopy
    return kvcopy


def _window_expected(src_t, src_addr, dst_addr, size, dst_base, lo, hi, sentinel):
    """Oracle image of dst bytes [lo, hi) (offsets from dst_base) after the one
    descriptor (src_addr, dst_addr, size), from the source bytes it reads."""
    img = np.full(hi - lo, sentinel, np.uint8)
    a = max(dst_base + lo, dst_addr)
    b = min(dst_base + hi, dst_addr + size)
    if a < b:
        s0 = src_addr + (a - dst_addr)
        src_off = s0 - src_t.data_ptr()
        s_img = src_t[src_off:src_off + (b - a)].cpu().numpy()
        oracle.copy([s0], [a], [b - a], [(s0, s_img)], [(dst_base + lo, img)])
    return img


@pytest.mark.parametrize("chunk", [0, 1 << 20])
def test_one_descriptor_over_4_gib(K, chunk):
    size = (5 << 30) + 8                      # ends in an odd 8-byte word
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    src = torch.randint(0, 256, (size + 64,), dtype=torch.uint8, device="cuda", generator=gen)
    dst = torch.full((size + 64,), W.SENTINEL_A, dtype=torch.uint8, device="cuda")
    src_addr, dst_addr = src.data_ptr() + 8, dst.data_ptr() + 16
    assert src_addr % 16 == 8 and dst_addr % 16 == 0
    _say("one descriptor of", size, "bytes, chunk", chunk or K.CHUNK_DEFAULT)
    K.kvcopy_batch([src_addr], [dst_addr], [size], K.D2D, 0, None, chunk_bytes=chunk)
    torch.cuda.synchronize()
    win = 1 << 16
    rng = np.random.default_rng(chunk)
    starts = [0, 16 + size - win + 48] + [16 + 8 * int(x) for x in
                                          rng.integers(0, (size - win) // 8, 64)]
    for lo in starts:
        hi = lo + win
        exp = _window_expected(src, src_addr, dst_addr, size, dst.data_ptr(), lo, hi, W.SENTINEL_A)
        got = dst[lo:hi].cpu().numpy()
        if not np.array_equal(got, exp):
            bad = int(np.flatnonzero(got != exp)[0])
            raise AssertionError(f"window at {lo}: first difference at dst offset {lo + bad}")
    del src, dst
    torch.cuda.empty_cache()


def test_a_million_descriptors(K):
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=9, n=1 << 20, max_size=128, dir_=W.H2D, src_where="host",
                     dst_where="device", misalign=True, zero_frac=0.01)
    res = Resident(wl)
    for max_wgs, chunk in ((0, 0), (64, 0), (0, 16)):
        _say("1,048,576 descriptors max_wgs", max_wgs, "chunk", chunk)
        res.fill()
        _run(res, [0], max_wgs, chunk_bytes=chunk)
        _check(res, [0], f"million descriptors max_wgs={max_wgs} chunk={chunk}")
    res.free()


@pytest.mark.parametrize("flags", [0, 2])
def test_adjacent_chain_coalesces_to_one_range(K, flags):
    """16,384 adjacent 4 KiB H2D descriptors: one merged 64 MiB range (4,096
    chunks) by default; 16,384 ranges with KVCOPY_F_NO_COALESCE (flags=2)."""
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=3, directions="h2d")
    b = wl.batches[0]
    n = 16384
    b.src_off[:] = np.arange(n, dtype=np.uint64) * 4096      # one run in both arenas
    b.dst_off[:] = np.uint64(4096 * 1000) + np.arange(n, dtype=np.uint64) * 4096
    res = Resident(wl)
    s, d = res.addrs[0]
    plan = K.kvcopy_plan(s, d, b.size)
    assert plan.n_merged == 1 and plan.n_chunks == n * 4096 // K.CHUNK_DEFAULT
    _say("adjacent chain flags", flags)
    _run(res, [0], 32, flags=flags)
    _check(res, [0], f"adjacent chain flags={flags}")
    res.free()
