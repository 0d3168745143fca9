"""GPU parity of kvcopy_batch_pair (two descriptor lists, one launch) against
the oracle, bit-exact.

The oracle applies list a and then list b with one memcpy per descriptor;
the lists touch disjoint bytes, so the order does not matter to the result.
Every case reads the touched arenas back whole (guard bytes included).
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import _check, _say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_copy_amd import kvcopy
    return kvcopy


def _pair(K, res, a, b, max_wgs, stream=None, **kw):
    """Submit batch a (or an empty list for None) and batch b in one call."""
    e = np.zeros(0, np.uint64)

    def lists(k):
        if k is None:
            return e, e, e
        s, d = res.addrs[k]
        return s, d, res.wl.batches[k].size

    st = getattr(stream, "cuda_stream", stream)
    return K.kvcopy_batch_pair(*lists(a), *lists(b), max_wgs, st, **kw)


@pytest.mark.parametrize("max_wgs", [1, 8, 128, 0, -1])
def test_pair_kv_bidirectional(K, max_wgs):
    """16,384 x 4 KiB H2D and D2H (the offload burst) in one launch."""
    from block_copy_amd.harness import Resident
    res = Resident(W.kv_blocks(seed=6, directions="both"))
    for a, b in ((0, 1), (1, 0)):
        _say("pair kv", "lists", a, b, "max_wgs", max_wgs)
        res.fill()
        _pair(K, res, a, b, max_wgs)
        torch.cuda.synchronize()
        _check(res, [0, 1], f"pair kv a={a} b={b} max_wgs={max_wgs}")
    res.free()


@pytest.mark.parametrize("max_wgs", [1, 3, 64, 0])
@pytest.mark.parametrize("na,nb", [(700, 37), (1, 2000), (129, 129), (5000, 1)])
def test_pair_unequal_irregular(K, na, nb, max_wgs):
    """Lists of very different chunk counts, misaligned, with zero sizes and
    ranges longer than a chunk: each wavefront's shares of the two lists
    differ in length and run out at different times."""
    from block_copy_amd.harness import Resident
    wl = W.combine("pair", W.irregular(seed=na, n=na, max_size=40 * 1024, dir_=W.H2D,
                                       src_where="host", misalign=True, zero_frac=0.05),
                   W.irregular(seed=nb + 1, n=nb, max_size=40 * 1024, dir_=W.D2H,
                               dst_where="host", misalign=True, zero_frac=0.05))
    res = Resident(wl)
    _say("pair irregular", na, nb, "max_wgs", max_wgs)
    _pair(K, res, 0, 1, max_wgs)
    torch.cuda.synchronize()
    _check(res, [0, 1], f"pair irregular na={na} nb={nb} max_wgs={max_wgs}")
    res.free()


@pytest.mark.parametrize("direction", ["h2d", "d2h"])
@pytest.mark.parametrize("side", ["a", "b"])
def test_pair_one_list_empty(K, side, direction):
    """One list only: every wavefront of the launch copies it."""
    from block_copy_amd.harness import Resident
    res = Resident(W.kv_blocks(seed=7, directions=direction, n=3000))
    for max_wgs in (1, 16, 0, -1):
        _say("pair one empty", side, direction, "max_wgs", max_wgs)
        res.fill()
        if side == "a":
            _pair(K, res, None, 0, max_wgs)
        else:
            _pair(K, res, 0, None, max_wgs)
        torch.cuda.synchronize()
        _check(res, [0], f"pair empty {side} {direction} max_wgs={max_wgs}")
    res.free()


def test_pair_d2d_with_h2d_and_flags(K):
    """Any direction in either list; validate mode and no-coalesce."""
    from block_copy_amd.harness import Resident
    wl = W.combine("pair", W.d2d_blocks(seed=3, n=2048),
                   W.h2d_mixed(seed=3, n=1500))
    res = Resident(wl)
    for flags in (0, K.F_VALIDATE, K.F_NO_COALESCE, K.F_VALIDATE | K.F_NO_COALESCE):
        for max_wgs in (2, 0):
            _say("pair d2d+h2d flags", flags, "max_wgs", max_wgs)
            res.fill()
            _pair(K, res, 0, 1, max_wgs, flags=flags)
            torch.cuda.synchronize()
            _check(res, [0, 1], f"pair d2d+h2d flags={flags} max_wgs={max_wgs}")
    res.free()


def test_pair_cross_list_overlap_rejected(K):
    """Validate mode sees across the lists: list b writing list a's
    destinations is rejected and nothing is enqueued (the arenas keep their
    fill)."""
    from block_copy_amd.harness import Resident
    res = Resident(W.kv_blocks(seed=8, directions="both", n=256, pool_blocks=2048))
    s0, d0 = res.addrs[0]
    z0 = res.wl.batches[0].size
    s1, _ = res.addrs[1]
    rc = K.kvcopy_batch_pair(s0, d0, z0, s1, d0, z0, 0, None, flags=K.F_VALIDATE, check=False)
    assert rc == K.EOVERLAP
    torch.cuda.synchronize()
    for i, a in enumerate(res.wl.arenas):
        assert np.array_equal(res.image(i), a.host_image()), f"arena {a.name} changed"
    res.free()


def test_pair_ring_reuse_and_mixed_calls(K):
    """Many pair calls and single-list calls on two streams: the staging
    ring wraps several times while earlier kernels may still read their
    records; the copies are idempotent, so the final images are the oracle's."""
    from block_copy_amd.harness import Resident
    res = Resident(W.kv_blocks(seed=9, directions="both"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _say("pair ring reuse: 40 pair calls + 40 single calls")
    for i in range(40):
        _pair(K, res, 0, 1, (1, 32, 128, 0)[i % 4], s1)
        res.submit(i % 2, (8, 0)[i % 2], s2)
    torch.cuda.synchronize()
    _check(res, [0, 1], "pair ring reuse")
    res.free()
