"""GPU parity: the HIP path through the C ABI against the oracle, bit-exact.

Every case builds the workload's arenas on the GPU (device memory, mapped
pinned host memory), runs kvcopy_batch, reads every touched arena back
whole (guard bytes included) and compares it with the oracle's image of the
same seeded inputs.  Several cases are repeated with a second sentinel so
that a payload byte equal to the sentinel cannot hide a skipped copy.
"""
import numpy as np
import pytest

import workloads as W
from expect import assert_same, expected_images

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

WGS = [1, 8, 32, 128, 0]


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_copy_amd import kvcopy
    return kvcopy


def _check(res, batch_ids, what, sentinel=None):
    wl = res.wl
    exp = expected_images(wl, batch_ids, res.bases, sentinel)
    for i, img in enumerate(exp):
        if img is None:
            continue
        bi = next((k for k in batch_ids if i in set(wl.batches[k].dst_arena.tolist())), None)
        assert_same(res.image(i), img, f"{what} arena {wl.arenas[i].name}", wl, bi, res.bases, i)


def _run(res, batch_ids, max_wgs, streams=None, **kw):
    if streams is None:
        for k in batch_ids:
            res.submit(k, max_wgs, None, **kw)
    else:
        for k, st in zip(batch_ids, streams):
            res.submit(k, max_wgs, st, **kw)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# D2D blocks: 1,024 x 4 KiB between two pools of 4,096 blocks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("max_wgs", WGS)
def test_d2d_blocks_full(K, max_wgs):
    from block_copy_amd.harness import Resident
    wl = W.d2d_blocks(seed=0)
    res = Resident(wl)
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        _say("d2d 1024x4KiB", "max_wgs", max_wgs, "sentinel", hex(sentinel))
        res.fill(sentinel)
        _run(res, [0], max_wgs)
        _check(res, [0], f"d2d max_wgs={max_wgs}", sentinel)
    res.free()


# ---------------------------------------------------------------------------
# H2D / D2H: 16,384 shuffled x 4 KiB against a 65,536-block pool
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("max_wgs", WGS)
@pytest.mark.parametrize("direction", ["h2d", "d2h"])
def test_kv_blocks_one_direction(K, direction, max_wgs):
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=1, directions=direction)
    res = Resident(wl)
    _say("kv", direction, "16384x4KiB max_wgs", max_wgs)
    _run(res, [0], max_wgs)
    _check(res, [0], f"{direction} max_wgs={max_wgs}")
    res.free()


@pytest.mark.parametrize("max_wgs", [8, 128, 0])
def test_kv_blocks_concurrent(K, max_wgs):
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=2, directions="both")
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        _say("kv both concurrent max_wgs", max_wgs, "sentinel", hex(sentinel))
        res.fill(sentinel)
        _run(res, [0, 1], max_wgs, streams=[s1, s2])
        _check(res, [0, 1], f"h2d+d2h max_wgs={max_wgs}", sentinel)
    res.free()


# ---------------------------------------------------------------------------
# H2D mixed sizes with partial adjacency (coalescing, 8-byte tails)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [16, 256, 4096, 65536])
def test_h2d_mixed(K, n):
    from block_copy_amd.harness import Resident
    wl = W.h2d_mixed(seed=3, n=n)
    res = Resident(wl)
    for max_wgs in ([1, 32, 0] if n <= 4096 else [64, 0]):
        _say("h2d mixed n", n, "max_wgs", max_wgs)
        res.fill()
        _run(res, [0], max_wgs)
        _check(res, [0], f"h2d mixed n={n} max_wgs={max_wgs}")
    res.free()


# ---------------------------------------------------------------------------
# MoE expert gather
# ---------------------------------------------------------------------------

def test_moe_gather_reduced_many_calls(K):
    """Successive calls on one stream (more calls than staging slots)."""
    from block_copy_amd.harness import Resident
    wl = W.moe_gather(seed=4, calls=12, n_experts=32, n_slots=96, misses=(5, 20))
    res = Resident(wl)
    _say("moe reduced 12 calls")
    _run(res, list(range(12)), 16)
    _check(res, list(range(12)), "moe reduced 12 calls")
    res.free()


def test_moe_gather_full_size(K):
    """256 experts x 6 banks on the host, 3,164 slots on the device (5.3 GB)."""
    from block_copy_amd.harness import Resident
    wl = W.moe_gather(seed=5, calls=3)
    res = Resident(wl)
    for max_wgs in (32, 0):
        _say("moe full size 3 calls max_wgs", max_wgs)
        res.fill()
        _run(res, [0, 1, 2], max_wgs)
        _check(res, [0, 1, 2], f"moe full max_wgs={max_wgs}")
    res.free()


# ---------------------------------------------------------------------------
# Irregular batches: misaligned (8 mod 16), zero sizes, shared sources,
# every direction, chunk sizes, flags
# ---------------------------------------------------------------------------

DIRS = {"d2d": (W.D2D, "device", "device"), "h2d": (W.H2D, "host", "device"),
        "d2h": (W.D2H, "device", "host")}


@pytest.mark.parametrize("dname", sorted(DIRS))
@pytest.mark.parametrize("chunk", [16, 1024, 4096, 16384, 65536, 1 << 20])
def test_irregular_chunk_sizes(K, dname, chunk):
    from block_copy_amd.harness import Resident
    d, sw, dw = DIRS[dname]
    wl = W.irregular(seed=chunk % 97, n=200, max_size=min(80 * 1024, 256 * chunk), dir_=d,
                     src_where=sw, dst_where=dw, misalign=True, zero_frac=0.05)
    res = Resident(wl)
    for max_wgs in (1, 7, 0):
        _say("irregular", dname, "chunk", chunk, "max_wgs", max_wgs)
        res.fill()
        _run(res, [0], max_wgs, chunk_bytes=chunk)
        _check(res, [0], f"irregular {dname} chunk={chunk} max_wgs={max_wgs}")
    res.free()


def test_kv_blocks_concurrent_on_dedicated_queues(K):
    """The headline burst on the streams bench.py uses: a hardware queue each
    (full CU mask), wrapped as torch streams."""
    from block_copy_amd import hiprt
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=4, directions="both")
    res = Resident(wl)
    q = hiprt.QueueStreams(2, torch.cuda.get_device_properties(0).multi_processor_count)
    try:
        for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
            _say("kv both on dedicated queues, sentinel", hex(sentinel))
            res.fill(sentinel)
            _run(res, [0, 1], 128, streams=q.streams)
            _check(res, [0, 1], f"h2d+d2h dedicated queues sentinel={sentinel:#x}", sentinel)
    finally:
        torch.cuda.synchronize()
        q.destroy()
        res.free()


@pytest.mark.parametrize("beside", ["alone", "h2d_other_stream", "h2d_same_stream"])
def test_d2h_store_forms(K, beside):
    """A D2H batch (sc1 stores) alone, beside an H2D kernel still running on
    another stream, and behind one on its own stream must leave the same
    bytes.  The D2H batch is irregular (misaligned pairs, 8-byte tails, zero
    sizes) and larger than the inline limit; the H2D batch is 16,384 x
    4 KiB, still running when the D2H batch is submitted."""
    from block_copy_amd.harness import Resident
    d2h = W.irregular(seed=61, n=600, dir_=W.D2H, src_where="device", dst_where="host",
                      misalign=True, zero_frac=0.05)
    wl = W.combine("d2h_beside_h2d", d2h, W.kv_blocks(seed=3, directions="h2d"))
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        _say("d2h store forms", beside, "sentinel", hex(sentinel))
        res.fill(sentinel)
        if beside == "alone":
            _run(res, [0], 128, streams=[s2])
            _check(res, [0], f"d2h alone sentinel={sentinel:#x}", sentinel)
            continue
        st = s1 if beside == "h2d_other_stream" else s2
        _run(res, [1, 0], 128, streams=[st, s2])
        _check(res, [0, 1], f"d2h {beside} sentinel={sentinel:#x}", sentinel)
    res.free()


@pytest.mark.parametrize("flags", [0, 1, 2, 8, 10, 11])
def test_irregular_flags(K, flags):
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=40 + flags, n=500, dir_=W.H2D, src_where="host", dst_where="device",
                     shared_src=(flags in (0, 8)))
    res = Resident(wl)
    _say("irregular flags", flags)
    _run(res, [0], 16, flags=flags)
    _check(res, [0], f"irregular flags={flags}")
    res.free()


def test_tiny_and_empty(K):
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=50, n=3, max_size=24, dir_=W.D2D)
    res = Resident(wl)
    _say("tiny and empty")
    assert K.kvcopy_batch([], [], [], K.D2D) == 0                       # n = 0
    s, d = res.addrs[0]
    assert K.kvcopy_batch(s, d, np.zeros(3, np.uint64), K.D2D) == 0     # only zero sizes
    torch.cuda.synchronize()
    for i, a in enumerate(wl.arenas):
        if a.fill == "sentinel":
            assert np.all(res.image(i) == a.sentinel)
    _run(res, [0], 0)
    _check(res, [0], "tiny")
    res.free()


def test_order_independence(K):
    """A shuffled descriptor list gives the same bytes (distinct destinations)."""
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=60, n=400, dir_=W.D2D)
    res = Resident(wl)
    b = wl.batches[0]
    perm = np.random.default_rng(0).permutation(b.n)
    s, d = res.addrs[0]
    _say("order independence")
    K.kvcopy_batch(s[perm], d[perm], b.size[perm], K.D2D, 8)
    torch.cuda.synchronize()
    _check(res, [0], "shuffled order")
    res.free()


def test_error_paths_enqueue_nothing(K):
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=70, n=50, dir_=W.D2D)
    res = Resident(wl)
    s, d = res.addrs[0]
    z = wl.batches[0].size.copy()
    _say("error paths")
    bad = z.copy()
    bad[7] += 4
    assert K.kvcopy_batch(s, d, bad, K.D2D, check=False) == K.EALIGN
    assert K.kvcopy_batch(s, d, z, 5, check=False) == K.EINVAL
    assert K.kvcopy_batch(s, d, z, K.D2D, -2, check=False) == K.EINVAL
    dd = d.copy()
    dd[3] = dd[2]                                     # two descriptors write the same bytes
    assert K.kvcopy_batch(s, dd, z, K.D2D, flags=K.F_VALIDATE, check=False) == K.EOVERLAP
    torch.cuda.synchronize()
    for i, a in enumerate(wl.arenas):
        if a.fill == "sentinel":
            assert np.all(res.image(i) == a.sentinel), "an error path enqueued work"
    res.free()


# ---------------------------------------------------------------------------
# The staging ring under load: wrap-around, growth, several host threads
# ---------------------------------------------------------------------------

def test_many_calls_wrap_the_staging_ring(K):
    """More worklist bytes queued than the ring holds: calls wait for ring
    space (kernels on two streams finish out of order) and every call still
    copies the right bytes."""
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=80, n=3000, max_size=4096, dir_=W.D2D)   # ~3,000 chunks = 72 KB of records
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _say("ring wrap: 600 calls on two streams")
    for i in range(600):                                              # ~43 MB of records > 16 MiB
        res.submit(0, 2 if i % 2 else 0, s1 if i % 2 else s2, flags=K.F_DESC_UPLOAD if i % 3 == 0 else 0)
    torch.cuda.synchronize()
    _check(res, [0], "after ring wrap")
    res.free()


def test_ring_regions_outlive_their_kernels(K):
    """Ring regions stay intact until their kernels have completed: see
    tests/ring_scenario.py.  It runs in a fresh process, where the library's
    staging ring has its initial 16 MiB (earlier tests in this process grow
    it past the size that the scenario must overfill)."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    _say("ring scenario in a fresh process")
    r = subprocess.run([sys.executable, os.path.join(here, "ring_scenario.py")],
                       capture_output=True, text=True, timeout=240)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_ring_growth_with_gpu_order_in_flight(K):
    """The ring grows while uploaded worklists and their order kernels are
    still queued: see tests/growth_scenario.py (a fresh process, so that the
    ring starts at 16 MiB and must grow)."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    _say("growth scenario in a fresh process")
    r = subprocess.run([sys.executable, os.path.join(here, "growth_scenario.py")],
                       capture_output=True, text=True, timeout=240)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_ring_growth_with_calls_in_flight(K):
    """A call whose worklist needs more than a quarter of the ring grows it
    while earlier calls are still queued."""
    from block_copy_amd.harness import Resident
    small = W.irregular(seed=81, n=500, max_size=8192, dir_=W.D2D)
    big = W.irregular(seed=82, n=240, max_size=32768, dir_=W.D2D)    # ~3.9 MB payload
    rs, rb = Resident(small), Resident(big)
    s1 = torch.cuda.Stream()
    _say("ring growth")
    for _ in range(20):
        rs.submit(0, 1, s1)
    rb.submit(0, 64, s1, chunk_bytes=16)          # 16-byte chunks: > 240 K records (> 4 MiB)
    for _ in range(5):
        rs.submit(0, 1, s1)
    torch.cuda.synchronize()
    _check(rs, [0], "small batch around ring growth")
    _check(rb, [0], "batch that grew the ring")
    rs.free()
    rb.free()


def test_threads_share_the_library(K):
    """Four host threads, each with its own stream and arenas, submit at once,
    cycling through the worklist's routes: read in place, uploaded, grouped
    by destination on the host, and uploaded and grouped on the GPU (the
    order kernels of all threads share the library's upload stream)."""
    import threading
    from block_copy_amd.harness import Resident
    wls = [W.irregular(seed=90 + t, n=400, max_size=16384, dir_=d, src_where=sw, dst_where=dw)
           for t, (d, sw, dw) in enumerate([DIRS["d2d"], DIRS["h2d"], DIRS["d2h"], DIRS["d2d"]])]
    rs = [Resident(wl) for wl in wls]
    streams = [torch.cuda.Stream() for _ in rs]
    errors = []

    def worker(t):
        try:
            routes = [0, K.F_DESC_UPLOAD, K.F_DST_ORDER, K.F_DST_ORDER | K.F_DESC_UPLOAD]
            for i in range(32):
                rs[t].submit(0, [0, 8, 32][i % 3], streams[t], flags=routes[(i + t) % 4])
        except Exception as e:   # noqa: BLE001 - reported below
            errors.append(e)

    _say("four threads")
    th = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t, r in enumerate(rs):
        _check(r, [0], f"thread {t}")
        r.free()



# ---------------------------------------------------------------------------
# Paced jobs: a batch in pieces, each submitted after the previous completed
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("piece", [0, 1, 7, 100, 2048])
def test_job_pieces_give_the_same_bytes(K, piece):
    import time
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=3, directions="both", n=2048, pool_blocks=8192)
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _say("job pieces", piece)
    jobs = []
    for j, st in ((0, s1), (1, s2)):
        s, d = res.addrs[j]
        jobs.append(K.kvcopy_job_create(s, d, wl.batches[j].size, wl.batches[j].dir, 16, piece,
                                        st.cuda_stream))
    pending = list(jobs)
    t0 = time.time()
    while pending:
        pending = [jb for jb in pending if not K.kvcopy_job_poll(jb)]
        assert time.time() - t0 < 60, "job did not finish"
    for jb in jobs:
        K.kvcopy_job_destroy(jb)
    torch.cuda.synchronize()
    _check(res, [0, 1], f"jobs piece={piece}")
    res.free()


def test_job_wait(K):
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=95, n=300, dir_=W.D2D)
    res = Resident(wl)
    s, d = res.addrs[0]
    _say("job wait")
    jb = K.kvcopy_job_create(s, d, wl.batches[0].size, K.D2D, 0, 32)
    K.kvcopy_job_wait(jb)
    assert K.kvcopy_job_poll(jb) is True
    K.kvcopy_job_destroy(jb)
    torch.cuda.synchronize()
    _check(res, [0], "job wait")
    res.free()



# ---------------------------------------------------------------------------
# KVCOPY_WGS_AUTO before and after the startup probe
# ---------------------------------------------------------------------------

def test_auto_cap_and_autotune(K):
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=4, directions="both", n=4096, pool_blocks=16384)
    res = Resident(wl)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _say("auto cap, default")
    _run(res, [0, 1], K.WGS_AUTO, streams=[s1, s2])
    _check(res, [0, 1], "WGS_AUTO default")
    _say("autotune")
    c1, r1 = K.kvcopy_autotune(K.H2D, s1.cuda_stream, s2.cuda_stream)
    c2, r2 = K.kvcopy_autotune(K.D2D)
    assert {c1, c2} <= set(K.AUTOTUNE_CAPS)
    assert all(v > 0 for v in list(r1.values()) + list(r2.values()))
    assert r1[c1] >= 0.98 * max(r1.values()) and r2[c2] >= 0.98 * max(r2.values())
    res.fill()
    _run(res, [0, 1], K.WGS_AUTO, streams=[s1, s2])
    _check(res, [0, 1], "WGS_AUTO tuned")
    res.free()


# ---------------------------------------------------------------------------
# CU-masked streams: the copy confined to a few compute units (the ROCm
# analogue of the Green Context SM limit in PegaFlow issue #408,
# "Follow-up", item 4)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n_cus", [8, 32])
def test_copies_on_cu_masked_streams(K, n_cus):
    """The headline burst (16,384 x 4 KiB each way, both directions on two
    streams) and an irregular D2D batch (misaligned pairs, 8-byte tails,
    zero sizes), each on streams whose kernels may use only the first
    n_cus compute units."""
    from block_copy_amd import hiprt
    from block_copy_amd.harness import Resident
    kv = Resident(W.kv_blocks(seed=6, directions="both"))
    irr = Resident(W.irregular(seed=7, n=3000, dir_=W.D2D, misalign=True, zero_frac=0.05))
    sa, sb = hiprt.CUMaskStream(range(n_cus)), hiprt.CUMaskStream(range(n_cus))
    try:
        for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
            for max_wgs in (8, 128):
                _say("cu-masked streams", n_cus, "CUs, max_wgs", max_wgs, "sentinel", hex(sentinel))
                kv.fill(sentinel)
                kv.submit(0, max_wgs, sa.cuda_stream)
                kv.submit(1, max_wgs, sb.cuda_stream)
                hiprt.stream_sync(sa)
                hiprt.stream_sync(sb)
                _check(kv, [0, 1], f"kv both on {n_cus} CUs max_wgs={max_wgs}", sentinel)
            irr.fill(sentinel)
            irr.submit(0, 0, sa.cuda_stream)
            hiprt.stream_sync(sa)
            _check(irr, [0], f"irregular d2d on {n_cus} CUs", sentinel)
    finally:
        torch.cuda.synchronize()
        sa.destroy()
        sb.destroy()
        kv.free()
        irr.free()


def test_kv_burst_on_cu_half_streams(K):
    """The headline's setting: H2D on a stream over the first half of the CU
    mask bits and D2H on one over the second half (each XCD keeps CUs for
    both), at the headline cap and at 8 and 128, several bursts back to back
    with the two streams joined per burst."""
    from block_copy_amd import hiprt
    from block_copy_amd.harness import Resident
    n = torch.cuda.get_device_properties(0).multi_processor_count
    kv = Resident(W.kv_blocks(seed=9, directions="both"))
    sa, sb = hiprt.CUMaskStream(range(n // 2), n), hiprt.CUMaskStream(range(n // 2, n), n)
    try:
        for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
            for max_wgs in (64, 8, 128):
                _say("cu-half streams, max_wgs", max_wgs, "sentinel", hex(sentinel))
                kv.fill(sentinel)
                for _ in range(5):
                    kv.submit(0, max_wgs, sa.cuda_stream)
                    kv.submit(1, max_wgs, sb.cuda_stream)
                    hiprt.stream_sync(sa)
                    hiprt.stream_sync(sb)
                _check(kv, [0, 1], f"kv both on CU halves max_wgs={max_wgs}", sentinel)
    finally:
        torch.cuda.synchronize()
        sa.destroy()
        sb.destroy()
        kv.free()


# ---------------------------------------------------------------------------
# Forced store forms, time-sliced issue, destination order
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("form", ["sc1", "nt"])
@pytest.mark.parametrize("dname", sorted(DIRS))
def test_forced_store_forms(K, dname, form):
    """KVCOPY_F_STORE_SC1 / KVCOPY_F_STORE_NT in every direction, through the
    staging ring (600 descriptors) and the inline worklist (40)."""
    from block_copy_amd.harness import Resident
    d, sw, dw = DIRS[dname]
    flag = K.F_STORE_SC1 if form == "sc1" else K.F_STORE_NT
    for n in (600, 40):
        wl = W.irregular(seed=100 + n + d, n=n, max_size=20000, dir_=d, src_where=sw, dst_where=dw,
                         misalign=True, zero_frac=0.05)
        res = Resident(wl)
        for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
            for max_wgs in (1, 16, 0):
                _say("store form", form, dname, "n", n, "max_wgs", max_wgs, "sentinel", hex(sentinel))
                res.fill(sentinel)
                _run(res, [0], max_wgs, flags=flag)
                _check(res, [0], f"{form} {dname} n={n} max_wgs={max_wgs}", sentinel)
        res.free()


def test_pair_nt_stores(K):
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=8, directions="both", n=4096, pool_blocks=16384)
    res = Resident(wl)
    (s0, d0), (s1, d1) = res.addrs
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        for max_wgs in (8, K.WGS_AUTO):
            _say("pair nt stores max_wgs", max_wgs, "sentinel", hex(sentinel))
            res.fill(sentinel)
            K.kvcopy_batch_pair(s0, d0, wl.batches[0].size, s1, d1, wl.batches[1].size, max_wgs,
                                flags=K.F_STORE_NT)
            torch.cuda.synchronize()
            _check(res, [0, 1], f"pair nt max_wgs={max_wgs}", sentinel)
    res.free()


@pytest.mark.parametrize("duty", [(2000, 10000), (1000, 50000), (10000, 10000)])
def test_duty_cycle(K, duty):
    """Time-sliced issue: both directions on two streams, and an irregular
    D2H batch with 8-byte tails, each kernel starting chunks only inside
    the on-windows.  (10 us of 10 us: the window covers the period.)"""
    from block_copy_amd.harness import Resident
    on, period = duty
    kv = Resident(W.kv_blocks(seed=9, directions="both", n=2048, pool_blocks=8192))
    irr = Resident(W.irregular(seed=10, n=500, dir_=W.D2H, src_where="device", dst_where="host",
                               misalign=True, zero_frac=0.05))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        for max_wgs in (2, 32):
            _say("duty cycle", on, period, "max_wgs", max_wgs, "sentinel", hex(sentinel))
            kv.fill(sentinel)
            _run(kv, [0, 1], max_wgs, streams=[s1, s2], duty_on_ns=on, duty_period_ns=period)
            _check(kv, [0, 1], f"duty {on}/{period} max_wgs={max_wgs}", sentinel)
        irr.fill(sentinel)
        _run(irr, [0], 4, duty_on_ns=on, duty_period_ns=period, flags=K.F_STORE_NT)
        _check(irr, [0], f"duty {on}/{period} irregular d2h", sentinel)
    kv.free()
    irr.free()


@pytest.mark.parametrize("max_wgs", [1, 64, 0])
def test_destination_order(K, max_wgs):
    """KVCOPY_F_DST_ORDER: the D2D block gather, an irregular batch whose
    ranges span several chunks (planned twice: more records than the first
    pass has room for), and an H2D batch."""
    from block_copy_amd.harness import Resident
    cases = [(W.d2d_blocks(seed=11), 0),
             (W.irregular(seed=12, n=700, max_size=80 * 1024, dir_=W.D2D, misalign=True,
                          zero_frac=0.05), 4096),
             (W.kv_blocks(seed=13, directions="h2d", n=4096, pool_blocks=16384), 0)]
    for wl, chunk in cases:
        res = Resident(wl)
        for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
            _say("destination order", wl.name, "max_wgs", max_wgs, "sentinel", hex(sentinel))
            res.fill(sentinel)
            _run(res, [0], max_wgs, flags=K.F_DST_ORDER, chunk_bytes=chunk)
            _check(res, [0], f"dst order {wl.name} max_wgs={max_wgs}", sentinel)
        res.free()


@pytest.mark.parametrize("loop", ["per_chunk", "pipeline", "dynamic", "wg"])
def test_destination_order_on_the_gpu(K, loop):
    """KVCOPY_F_DST_ORDER | KVCOPY_F_DESC_UPLOAD: the worklist is uploaded in
    list order and grouped by destination region by two kernels on the
    call's stream before the copy.  Record counts around the order kernels'
    workgroup share (1,024 records) and thread count (256), the D2D block
    gather, an irregular misaligned batch with multi-chunk ranges and zero
    sizes, and H2D and D2H batches; each loop reads the ordered copy."""
    from block_copy_amd.harness import Resident
    extra = {"per_chunk": 0, "pipeline": K.F_PIPELINE, "dynamic": K.F_DYNAMIC,
             "wg": K.F_WG_PER_CHUNK}[loop]
    fl = K.F_DST_ORDER | K.F_DESC_UPLOAD | extra
    cases = [(W.d2d_blocks(seed=30 + i, n=n, pool_blocks=8192, block=64), 0)
             for i, n in enumerate((1, 2, 255, 256, 257, 1023, 1024, 1025, 4097))]
    cases += [(W.d2d_blocks(seed=41), 0),
              (W.irregular(seed=42, n=900, max_size=80 * 1024, dir_=W.D2D, misalign=True,
                           zero_frac=0.05), 4096),
              (W.kv_blocks(seed=43, directions="h2d", n=4096, pool_blocks=16384), 0),
              (W.irregular(seed=44, n=700, dir_=W.D2H, src_where="device", dst_where="host",
                           misalign=True, zero_frac=0.05), 0)]
    for wl, chunk in cases:
        res = Resident(wl)
        for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
            for max_wgs in (8, 0):
                _say("gpu destination order", loop, wl.name, "n", wl.batches[0].n, "max_wgs",
                     max_wgs, "sentinel", hex(sentinel))
                res.fill(sentinel)
                _run(res, [0], max_wgs, flags=fl, chunk_bytes=chunk)
                _check(res, [0], f"gpu dst order {loop} {wl.name} n={wl.batches[0].n} "
                       f"max_wgs={max_wgs}", sentinel)
        res.free()


def test_destination_order_on_the_gpu_grid_stride(K):
    """More records than the order kernels' largest grid covers in one pass
    (1,024 workgroups x 1,024 records): 1,200,000 blocks of 64 bytes, so
    each order workgroup strides over the worklist twice."""
    from block_copy_amd.harness import Resident
    wl = W.d2d_blocks(seed=45, n=1_200_000, pool_blocks=1_400_000, block=64)
    res = Resident(wl)
    for loop_flag in (0, K.F_WG_PER_CHUNK):
        _say("gpu destination order, 1,200,000 records, loop flag", hex(loop_flag))
        res.fill(W.SENTINEL_A)
        _run(res, [0], 0, flags=K.F_DST_ORDER | K.F_DESC_UPLOAD | loop_flag)
        _check(res, [0], f"gpu dst order 1.2M records loop={hex(loop_flag)}", W.SENTINEL_A)
    res.free()


def test_tail_bounded_preset(K):
    """KVCOPY_F_TAIL_BOUNDED (sc1 stores, time-sliced issue, at most 4
    workgroups): the KV burst on two streams, an irregular D2H batch, and
    the preset with the nt store form and with its own duty cycle."""
    from block_copy_amd.harness import Resident
    kv = Resident(W.kv_blocks(seed=14, directions="both", n=2048, pool_blocks=8192))
    irr = Resident(W.irregular(seed=15, n=400, dir_=W.D2H, src_where="device", dst_where="host",
                               misalign=True, zero_frac=0.05))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    cases = [dict(flags=K.F_TAIL_BOUNDED), dict(flags=K.F_TAIL_BOUNDED | K.F_STORE_NT),
             dict(flags=K.F_TAIL_BOUNDED, duty_on_ns=1000, duty_period_ns=5000)]
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        for kw in cases:
            _say("tail-bounded", kw, "sentinel", hex(sentinel))
            kv.fill(sentinel)
            _run(kv, [0, 1], K.WGS_AUTO, streams=[s1, s2], **kw)
            _check(kv, [0, 1], f"tail-bounded {kw}", sentinel)
            irr.fill(sentinel)
            _run(irr, [0], 0, **kw)
            _check(irr, [0], f"tail-bounded irregular {kw}", sentinel)
    kv.free()
    irr.free()
