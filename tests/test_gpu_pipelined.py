"""GPU parity of the pipelined copy loop (KVCOPY_F_PIPELINE) against the oracle.

The pipelined loop streams each wavefront's chunks as 4 KiB pieces, two
16 KiB passes in flight, with pieces of one pass drawn from different chunks
and 8-byte tails riding in the same pass.  Every case reads the touched
arenas back whole (guard bytes included) and compares them bit-exact with
the oracle's images of the same seeded inputs.
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


@pytest.mark.parametrize("max_wgs", [1, 4])
@pytest.mark.parametrize("direction", ["h2d", "d2h"])
def test_per_chunk_loop_forced_on_small_grids(K, direction, max_wgs):
    """Small grids pick the pipelined loop by default; the per-chunk loop must
    still give the same bytes when forced."""
    from block_copy_amd.harness import Resident
    wl = W.kv_blocks(seed=5, directions=direction)
    res = Resident(wl)
    _say("per-chunk forced", direction, "max_wgs", max_wgs)
    _run(res, [0], max_wgs, flags=K.F_PER_CHUNK)
    _check(res, [0], f"per-chunk {direction} max_wgs={max_wgs}")
    res.free()
