"""GPU parity of every copy loop against the oracle, bit-exact.

- pipelined (KVCOPY_F_PIPELINE, and the default for small D2D grids): each
  wavefront streams its chunks as 4 KiB pieces, two 16 KiB passes in flight,
  pieces of one pass drawn from different chunks, 8-byte tails in the same
  pass;
- per-chunk forced where the default would pick the pipelined loop;
- dynamic claims (KVCOPY_F_DYNAMIC): chunks claimed with device atomics,
  counters reset by each kernel's last wavefront;
- one workgroup per chunk (KVCOPY_F_WG_PER_CHUNK): the four wavefronts of a
  workgroup share each chunk;
- inline worklists (the default for batches of at most 128 chunks): the
  records travel in the kernel arguments.
Every case reads the touched arenas back whole (guard bytes included) and
compares them with the oracle's images of the same seeded inputs.
"""
import pytest

import workloads as W
from test_gpu_parity import DIRS, _check, _run, _say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_copy_amd import kvcopy
    return kvcopy


@pytest.mark.parametrize("dname", sorted(DIRS))
@pytest.mark.parametrize("chunk", [16, 1024, 4096, 16384, 1 << 20])
def test_pipelined_irregular(K, dname, chunk):
    """src != dst mod 16, 8-byte tails, zero sizes; pieces shorter than a row."""
    from block_copy_amd.harness import Resident
    d, sw, dw = DIRS[dname]
    wl = W.irregular(seed=chunk % 89 + 7, n=300, max_size=min(80 * 1024, 256 * chunk), dir_=d,
                     src_where=sw, dst_where=dw, misalign=True, zero_frac=0.05)
    res = Resident(wl)
    for max_wgs in (1, 3, 0):
        _say("pipelined irregular", dname, "chunk", chunk, "max_wgs", max_wgs)
        res.fill()
        _run(res, [0], max_wgs, chunk_bytes=chunk, flags=K.F_PIPELINE)
        _check(res, [0], f"pipelined irregular {dname} chunk={chunk} max_wgs={max_wgs}")
    res.free()


@pytest.mark.parametrize("max_wgs", [1, 8, 128, 0])
def test_pipelined_d2d_blocks(K, max_wgs):
    from block_copy_amd.harness import Resident
    wl = W.d2d_blocks(seed=0)
    res = Resident(wl)
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        _say("pipelined d2d 1024x4KiB max_wgs", max_wgs, "sentinel", hex(sentinel))
        res.fill(sentinel)
        _run(res, [0], max_wgs, flags=K.F_PIPELINE)
        _check(res, [0], f"pipelined d2d max_wgs={max_wgs}", sentinel)
    res.free()


@pytest.mark.parametrize("max_wgs", [1, 16, 128, 0])
def test_pipelined_kv_concurrent(K, max_wgs):
    """16,384 x 4 KiB each way on two streams: more than 64 chunks per wavefront at small caps."""
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=2, directions="both")
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _say("pipelined kv both max_wgs", max_wgs)
    _run(res, [0, 1], max_wgs, streams=[s1, s2], flags=K.F_PIPELINE)
    _check(res, [0, 1], f"pipelined h2d+d2h max_wgs={max_wgs}")
    res.free()


@pytest.mark.parametrize("n", [16, 4096, 65536])
def test_pipelined_h2d_mixed(K, n):
    from block_copy_amd.harness import Resident
    wl = W.h2d_mixed(seed=3, n=n)
    res = Resident(wl)
    for max_wgs in (2, 64, 0):
        _say("pipelined h2d mixed n", n, "max_wgs", max_wgs)
        res.fill()
        _run(res, [0], max_wgs, flags=K.F_PIPELINE)
        _check(res, [0], f"pipelined h2d mixed n={n} max_wgs={max_wgs}")
    res.free()


def test_pipelined_moe_reduced(K):
    from block_copy_amd.harness import Resident
    wl = W.moe_gather(seed=4, calls=6, n_experts=32, n_slots=96, misses=(5, 20))
    res = Resident(wl)
    _say("pipelined moe reduced 6 calls")
    _run(res, list(range(6)), 8, flags=K.F_PIPELINE)
    _check(res, list(range(6)), "pipelined moe reduced")
    res.free()


def test_pipelined_d2d_large_chunks_and_upload(K):
    """65,536 x 4 KiB between 1 GiB pools with the worklist uploaded to device memory."""
    from block_copy_amd.harness import Resident
    wl = W.d2d_blocks(seed=1, n=65536, pool_blocks=262144)
    res = Resident(wl)
    for max_wgs, flags in ((512, K.F_PIPELINE), (2048, K.F_PIPELINE | K.F_DESC_UPLOAD)):
        _say("pipelined d2d 65536x4KiB max_wgs", max_wgs, "flags", flags)
        res.fill()
        _run(res, [0], max_wgs, flags=flags)
        _check(res, [0], f"pipelined d2d 65536 max_wgs={max_wgs} flags={flags}")
    res.free()


@pytest.mark.parametrize("max_wgs", [1, 64])
def test_per_chunk_loop_forced_on_small_d2d_grids(K, max_wgs):
    """Small D2D grids pick the pipelined loop by default; the per-chunk loop
    must still give the same bytes when forced."""
    from block_copy_amd.harness import Resident
    wl = W.d2d_blocks(seed=5)
    res = Resident(wl)
    _say("per-chunk forced d2d max_wgs", max_wgs)
    _run(res, [0], max_wgs, flags=K.F_PER_CHUNK)
    _check(res, [0], f"per-chunk d2d max_wgs={max_wgs}")
    res.free()


# ---------------------------------------------------------------------------
# Dynamic claiming (KVCOPY_F_DYNAMIC): chunks claimed with device atomics
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dname", sorted(DIRS))
@pytest.mark.parametrize("chunk", [16, 4096, 16384])
def test_dynamic_irregular(K, dname, chunk):
    from block_copy_amd.harness import Resident
    d, sw, dw = DIRS[dname]
    wl = W.irregular(seed=chunk % 83 + 11, n=300, max_size=min(80 * 1024, 256 * chunk), dir_=d,
                     src_where=sw, dst_where=dw, misalign=True, zero_frac=0.05)
    res = Resident(wl)
    for max_wgs in (1, 5, 0):
        _say("dynamic irregular", dname, "chunk", chunk, "max_wgs", max_wgs)
        res.fill()
        _run(res, [0], max_wgs, chunk_bytes=chunk, flags=K.F_DYNAMIC)
        _check(res, [0], f"dynamic irregular {dname} chunk={chunk} max_wgs={max_wgs}")
    res.free()


@pytest.mark.parametrize("max_wgs", [1, 8, 128, 0])
def test_dynamic_kv_concurrent(K, max_wgs):
    """Two calls in flight at once on two streams, each with its own counters."""
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=6, directions="both")
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _say("dynamic kv both max_wgs", max_wgs)
    _run(res, [0, 1], max_wgs, streams=[s1, s2], flags=K.F_DYNAMIC)
    _check(res, [0, 1], f"dynamic h2d+d2h max_wgs={max_wgs}")
    res.free()


def test_dynamic_counters_reset_across_many_calls(K):
    """Every call must find its claim counters at zero.  (a) 100 KV bursts
    (393 KiB of worklist each, so the 16 MiB staging ring wraps twice), H2D
    on one stream and D2H on another, dynamic and static calls mixed; every
    burst writes the same bytes, so the final images are those of one burst.
    (b) 40 MoE gathers with different slots on one stream, in order."""
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=8, directions="both")
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _say("dynamic: 100 kv bursts on two streams, mixed with static calls")
    for i in range(100):
        flags = K.F_DYNAMIC if i % 3 else 0
        res.submit(i % 2, (1, 4, 16, 0)[(i // 2) % 4], s1 if i % 2 else s2, flags=flags)
    torch.cuda.synchronize()
    _check(res, [0, 1], "dynamic kv bursts")
    res.free()
    wl = W.moe_gather(seed=7, calls=40, n_experts=24, n_slots=80, misses=(3, 12))
    res = Resident(wl)
    st = torch.cuda.Stream()
    _say("dynamic: 40 moe calls on one stream")
    for i in range(40):
        res.submit(i, (1, 4, 16, 0)[i % 4], st, flags=K.F_DYNAMIC if i % 3 else 0)
    torch.cuda.synchronize()
    _check(res, list(range(40)), "dynamic moe calls")
    res.free()


def test_dynamic_d2d_large(K):
    from block_copy_amd.harness import Resident
    wl = W.d2d_blocks(seed=1, n=65536, pool_blocks=262144)
    res = Resident(wl)
    for max_wgs in (512, 0):
        _say("dynamic d2d 65536x4KiB max_wgs", max_wgs)
        res.fill()
        _run(res, [0], max_wgs, flags=K.F_DYNAMIC)
        _check(res, [0], f"dynamic d2d 65536 max_wgs={max_wgs}")
    res.free()


# ---------------------------------------------------------------------------
# One workgroup per chunk (KVCOPY_F_WG_PER_CHUNK): the four wavefronts of a
# workgroup share each chunk, 4 KiB rows, the record read by the workgroup
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dname", sorted(DIRS))
@pytest.mark.parametrize("chunk", [16, 1024, 4096, 16384, 1 << 20])
def test_wg_per_chunk_irregular(K, dname, chunk):
    """Chunks shorter than a 4 KiB row, rows cut short, passes of 16 KiB,
    8-byte tails, src != dst mod 16, zero sizes; grids below and at the chunk
    count, the worklist in pinned memory, uploaded and in destination order,
    in both store forms."""
    from block_copy_amd.harness import Resident
    d, sw, dw = DIRS[dname]
    wl = W.irregular(seed=chunk % 97 + 5, n=300, max_size=min(80 * 1024, 256 * chunk), dir_=d,
                     src_where=sw, dst_where=dw, misalign=True, zero_frac=0.05)
    res = Resident(wl)
    for max_wgs, extra in ((1, 0), (7, K.F_DESC_UPLOAD), (0, 0),
                           (0, K.F_DESC_UPLOAD | K.F_STORE_SC1), (5, K.F_DST_ORDER | K.F_STORE_NT)):
        _say("wg-per-chunk irregular", dname, "chunk", chunk, "max_wgs", max_wgs, "flags", extra)
        res.fill()
        _run(res, [0], max_wgs, chunk_bytes=chunk, flags=K.F_WG_PER_CHUNK | extra)
        _check(res, [0], f"wg-per-chunk irregular {dname} chunk={chunk} max_wgs={max_wgs} "
                         f"flags={extra}")
    res.free()


@pytest.mark.parametrize("max_wgs", [1, 64, 0])
def test_wg_per_chunk_d2d_blocks(K, max_wgs):
    from block_copy_amd.harness import Resident
    wl = W.d2d_blocks(seed=0)
    res = Resident(wl)
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        for extra in (0, K.F_DESC_UPLOAD | K.F_DST_ORDER):
            _say("wg-per-chunk d2d 1024x4KiB max_wgs", max_wgs, "flags", extra, "sentinel",
                 hex(sentinel))
            res.fill(sentinel)
            _run(res, [0], max_wgs, flags=K.F_WG_PER_CHUNK | extra)
            _check(res, [0], f"wg-per-chunk d2d max_wgs={max_wgs} flags={extra}", sentinel)
    res.free()


def test_wg_per_chunk_d2d_large(K):
    """65,536 x 4 KiB between two 1 GiB pools: one workgroup per chunk, and a
    capped grid whose workgroups stride over the chunks."""
    from block_copy_amd.harness import Resident
    wl = W.d2d_blocks(seed=1, n=65536, pool_blocks=262144)
    res = Resident(wl)
    for max_wgs in (0, 4096):
        _say("wg-per-chunk d2d 65536x4KiB max_wgs", max_wgs)
        res.fill()
        _run(res, [0], max_wgs, flags=K.F_WG_PER_CHUNK | K.F_DESC_UPLOAD | K.F_DST_ORDER)
        _check(res, [0], f"wg-per-chunk d2d 65536 max_wgs={max_wgs}")
    res.free()


@pytest.mark.parametrize("loop", ["per_chunk", "wg", "per_chunk_dst_order", "wg_dst_order"])
def test_upload_train_wraps_the_ring(K, loop):
    """48 uploaded calls back to back on one stream, cycling over 8 batches
    of 16,384 random 4 KiB blocks (393 KiB of worklist each: the 16 MiB
    staging ring and its device twin wrap), so each call's worklist copy,
    on the library's upload stream, runs while earlier kernels still read
    their own regions; with destination order each call also runs the two
    order kernels on its region's header and ordered copy.  The pools'
    sources are never written, so the final images are those of the 8
    batches applied once, in order."""
    from block_copy_amd.harness import Resident
    wl = W.d2d_rotation(n=16384, pool_blocks=65536)
    res = Resident(wl)
    fl = K.F_DESC_UPLOAD | (K.F_WG_PER_CHUNK if loop.startswith("wg") else 0)
    if loop.endswith("dst_order"):
        fl |= K.F_DST_ORDER
    st = torch.cuda.Stream()
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        _say("upload train", loop, "sentinel", hex(sentinel))
        res.fill(sentinel)
        for i in range(48):
            res.submit(i % 8, 0, st, flags=fl)
        torch.cuda.synchronize()
        _check(res, list(range(8)), f"upload train {loop}", sentinel)
    res.free()


@pytest.mark.parametrize("max_wgs", [8, 0])
def test_wg_per_chunk_kv_concurrent(K, max_wgs):
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=6, directions="both")
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _say("wg-per-chunk kv both max_wgs", max_wgs)
    _run(res, [0, 1], max_wgs, streams=[s1, s2], flags=K.F_WG_PER_CHUNK)
    _check(res, [0, 1], f"wg-per-chunk h2d+d2h max_wgs={max_wgs}")
    res.free()


# ---------------------------------------------------------------------------
# Inline worklists: batches of at most 128 chunks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dname", sorted(DIRS))
@pytest.mark.parametrize("case", ["one", "few", "full", "tiny_chunks"])
def test_inline_worklist(K, dname, case):
    """Small batches whose chunk bound fits the kernel arguments: 1 descriptor,
    a few, a batch close to the 128-record limit, and 16-byte chunks."""
    from block_copy_amd.harness import Resident
    d, sw, dw = DIRS[dname]
    n, max_size, chunk = {"one": (1, 16 * 1024, 0), "few": (7, 40 * 1024, 0),
                          "full": (60, 16 * 1024, 0), "tiny_chunks": (20, 64, 16)}[case]
    wl = W.irregular(seed=len(case) * 7 + n, n=n, max_size=max_size, dir_=d, src_where=sw,
                     dst_where=dw, misalign=True, zero_frac=0.1 if n > 1 else 0.0)
    res = Resident(wl)
    s, dd = res.addrs[0]
    pl = K.kvcopy_plan(s, dd, wl.batches[0].size, chunk)
    assert pl.n_chunks <= 128
    for max_wgs in (1, 2, 0):
        _say("inline", dname, case, "chunks", pl.n_chunks, "max_wgs", max_wgs)
        res.fill()
        _run(res, [0], max_wgs, chunk_bytes=chunk)
        _check(res, [0], f"inline {dname} {case} max_wgs={max_wgs}")
    res.free()


def test_inline_and_ring_calls_interleaved(K):
    """Small (inline) and large (staging ring) batches alternating on two streams."""
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=9, directions="both")
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    (hs, hd), (ds, dd) = res.addrs
    z = wl.batches[0].size
    _say("inline and ring calls interleaved")
    for i in range(0, 16384, 1024):
        K.kvcopy_batch(hs[i:i + 1024], hd[i:i + 1024], z[i:i + 1024], K.H2D, 8, s1.cuda_stream)
        for j in range(i, i + 1024, 64):       # 64 blocks = 64 chunks: inline
            K.kvcopy_batch(ds[j:j + 64], dd[j:j + 64], z[j:j + 64], K.D2H, 0, s2.cuda_stream)
    torch.cuda.synchronize()
    _check(res, [0, 1], "inline and ring interleaved")
    res.free()
