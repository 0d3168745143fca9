"""The no-allocation entry point (kvcopy_batch_device_noalloc) against the
device-resident entry point it varies (kvcopy_batch_device, with a
caller-allocated workspace) and against the oracle.

Calls follow each other on one stream and share the library's workspace
array, each smaller than the one before (the first at the largest max_n the
array holds), so a stale word from an earlier call would show.  Every call
runs the same descriptors through both entry points on two identical sets
of arenas; the two destination arenas must be equal byte for byte, and
equal to the oracle's image."""
import numpy as np
import pytest

import workloads as W
from expect import assert_same, expected_images

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_copy_amd import kvcopy
    return kvcopy


def _dev_u64(a, pad_to=None, pad_value=0):
    a = np.asarray(a, dtype=np.uint64)
    if pad_to is not None and pad_to > a.size:
        a = np.concatenate([a, np.full(pad_to - a.size, pad_value, np.uint64)])
    return torch.from_numpy(a.view(np.int64).copy()).to("cuda")


def _u64(t):
    return int(t.cpu().numpy().view(np.uint64)[0])


def _call_pair(K, wl, max_n, max_wgs, chunk, status_want=0):
    """One call through each entry point on its own copy of the arenas."""
    from block_copy_amd.harness import Resident
    ra, rb = Resident(wl), Resident(wl)
    b = wl.batches[0]
    lists = []
    for r in (ra, rb):
        s, d = r.addrs[0]
        # entries past the count hold valid addresses (a stray read would
        # copy wrong bytes, which the comparison catches, not fault)
        lists.append((_dev_u64(s, max_n, int(s[0])), _dev_u64(d, max_n, int(d[0])),
                      _dev_u64(b.size, max_n, 8), _dev_u64([b.n])))
    ws = torch.empty(K.kvcopy_device_workspace_bytes(max_n) + 256, dtype=torch.uint8, device="cuda")
    base = (ws.data_ptr() + 255) // 256 * 256
    status = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    (sa, da, za, na), (sb, db, zb, nb) = lists
    K.kvcopy_batch_device(sa.data_ptr(), da.data_ptr(), za.data_ptr(), na.data_ptr(), max_n,
                          b.dir, max_wgs, base, chunk_bytes=chunk)
    K.kvcopy_batch_device_noalloc(sb.data_ptr(), db.data_ptr(), zb.data_ptr(), nb.data_ptr(), max_n,
                                  b.dir, max_wgs, status.data_ptr(), chunk_bytes=chunk)
    torch.cuda.synchronize()
    ws_status = int(ws[base - ws.data_ptr():base - ws.data_ptr() + 8].cpu().numpy().view(np.uint64)[0])
    assert ws_status == status_want
    assert _u64(status) == status_want
    dst = int(b.dst_arena[0])
    got_a, got_b = ra.image(dst), rb.image(dst)
    assert_same(got_b, got_a, f"{wl.name}: no-allocation call vs caller-workspace call")
    if status_want == 0:
        exp = expected_images(wl, [0], rb.bases)
        assert_same(got_b, exp[dst], f"{wl.name}: no-allocation call vs oracle")
    else:   # a rejected batch copies nothing
        assert np.all(got_b == wl.arenas[dst].sentinel)
    ra.free()
    rb.free()


@pytest.mark.parametrize("dname", ["d2d", "h2d"])
def test_calls_in_a_row_shrinking(K, dname):
    d, sw, dw = {"d2d": (W.D2D, "device", "device"), "h2d": (W.H2D, "host", "device")}[dname]
    big = W.d2d_blocks(seed=21, n=K.NOALLOC_MAX_N, pool_blocks=2 * K.NOALLOC_MAX_N, block=512)
    if dname == "h2d":
        big = W.kv_blocks(seed=22, directions="h2d", n=K.NOALLOC_MAX_N,
                          pool_blocks=2 * K.NOALLOC_MAX_N, block=512)
    mid = W.irregular(seed=23, n=3000, max_size=40 * 1024, dir_=d, src_where=sw, dst_where=dw,
                      misalign=True, zero_frac=0.05)
    small = W.irregular(seed=24, n=300, max_size=20 * 1024, dir_=d, src_where=sw, dst_where=dw,
                        misalign=True, zero_frac=0.05)
    for wl, max_n, max_wgs, chunk in ((big, K.NOALLOC_MAX_N, 0, 0), (mid, 4000, 64, 4096),
                                      (small, 300, 8, 0)):
        _say("no-alloc", dname, wl.name, "max_n", max_n, "max_wgs", max_wgs, "chunk", chunk)
        _call_pair(K, wl, max_n, max_wgs, chunk)


def test_misaligned_batch_reports_status(K):
    wl = W.irregular(seed=25, n=200, dir_=W.D2D, misalign=True)
    wl.batches[0].size[17] += 4                       # not a multiple of 8
    _say("no-alloc misaligned status")
    _call_pair(K, wl, 200, 16, 0, status_want=K.DEVICE_BAD_ALIGN)
    good = W.irregular(seed=26, n=150, dir_=W.D2D, misalign=True)
    _say("no-alloc after a rejected batch")
    _call_pair(K, good, 150, 16, 0)


def test_argument_errors_enqueue_nothing(K):
    x = torch.zeros(4, dtype=torch.int64, device="cuda")
    p = x.data_ptr()
    assert K.kvcopy_batch_device_noalloc(p, p, p, p, K.NOALLOC_MAX_N + 1, W.D2D, 8,
                                         check=False) == K.EINVAL
    assert K.kvcopy_batch_device_noalloc(p, p, p, p, 4, 7, 8, check=False) == K.EINVAL
    assert K.kvcopy_batch_device_noalloc(p, p, p, p, 4, W.D2D, -2, check=False) == K.EINVAL
    assert K.kvcopy_batch_device_noalloc(p, p, p, p, 4, W.D2D, 8, chunk_bytes=24,
                                         check=False) == K.EINVAL
    assert K.kvcopy_batch_device_noalloc(0, p, p, p, 4, W.D2D, 8, check=False) == K.EINVAL
    assert K.kvcopy_batch_device_noalloc(0, 0, 0, 0, 0, W.D2D, 8, check=False) == K.OK
