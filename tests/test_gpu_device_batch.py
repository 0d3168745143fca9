"""GPU parity of the device-resident batch (kvcopy_batch_device): descriptor
arrays and count in device memory, fixed launch shapes, HIP-graph capture.
Every result is compared bit-exact with the oracle's image of the same
inputs (tests/expect.py)."""
import numpy as np
import pytest

import oracle
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


def _workspace(K, max_n):
    nb = K.kvcopy_device_workspace_bytes(max_n)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device="cuda")
    base = (ws.data_ptr() + 255) // 256 * 256
    return ws, base


def _status(base):
    import ctypes
    from block_copy_amd import hiprt
    out = np.zeros(1, np.uint64)
    rc = hiprt.hip.hipMemcpy(ctypes.c_void_p(out.ctypes.data), ctypes.c_void_p(base), 8, 2)
    assert rc == 0
    return int(out[0])


DIRS = {"d2d": (W.D2D, "device", "device"), "h2d": (W.H2D, "host", "device"),
        "d2h": (W.D2H, "device", "host")}


@pytest.mark.parametrize("dname", sorted(DIRS))
@pytest.mark.parametrize("chunk", [16, 4096, 16384, 1 << 20])
def test_device_batch_matches_oracle(K, dname, chunk):
    from block_copy_amd.harness import Resident
    d, sw, dw = DIRS[dname]
    wl = W.irregular(seed=7 + chunk % 13, n=300, max_size=min(40 * 1024, 512 * chunk), dir_=d,
                     src_where=sw, dst_where=dw, zero_frac=0.05)
    res = Resident(wl)
    b = wl.batches[0]
    s, dd = res.addrs[0]
    max_n = 400
    # Entries past the count must not be read.  They hold valid addresses (a
    # stray read would not fault) that would overwrite the first 8 bytes of
    # descriptor 0's destination with other source bytes, which the
    # comparison would catch.
    ds, dt, dz = (_dev_u64(s, max_n, res.bases[0] + 8), _dev_u64(dd, max_n, int(dd[0])),
                  _dev_u64(b.size, max_n, 8))
    dn = _dev_u64([b.n])
    ws, base = _workspace(K, max_n)
    for max_wgs in (1, 16, 0):
        _say("device batch", dname, "chunk", chunk, "max_wgs", max_wgs)
        res.fill()
        K.kvcopy_batch_device(ds.data_ptr(), dt.data_ptr(), dz.data_ptr(), dn.data_ptr(), max_n, d,
                              max_wgs, base, chunk_bytes=chunk)
        torch.cuda.synchronize()
        assert _status(base) == 0
        exp = expected_images(wl, [0], res.bases)
        assert_same(res.image(1), exp[1], f"device batch {dname} chunk={chunk} max_wgs={max_wgs}")
    res.free()


def test_device_count_is_clamped_to_max_n(K):
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=31, n=200, dir_=W.D2D)
    res = Resident(wl)
    b = wl.batches[0]
    s, d = res.addrs[0]
    max_n = 150
    dn = _dev_u64([10**9])
    ws, base = _workspace(K, max_n)
    # keep the device arrays referenced until the kernels have run: a
    # temporary's memory goes back to torch's allocator at once
    ds, dt, dz = _dev_u64(s), _dev_u64(d), _dev_u64(b.size)
    _say("device count clamp")
    K.kvcopy_batch_device(ds.data_ptr(), dt.data_ptr(), dz.data_ptr(), dn.data_ptr(), max_n,
                          W.D2D, 8, base)
    torch.cuda.synchronize()
    exp = np.full(wl.arenas[1].nbytes, wl.arenas[1].sentinel, np.uint8)
    oracle.copy(s[:max_n], d[:max_n], b.size[:max_n], [(res.bases[0], wl.arenas[0].host_image())],
                [(res.bases[1], exp)])
    assert_same(res.image(1), exp, "clamped count")
    res.free()


def test_device_misaligned_descriptor_copies_nothing(K):
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=32, n=100, dir_=W.D2D)
    res = Resident(wl)
    b = wl.batches[0]
    s, d = res.addrs[0]
    z = b.size.copy()
    z[57] += 4
    ws, base = _workspace(K, 100)
    ds, dt, dz, dn = _dev_u64(s), _dev_u64(d), _dev_u64(z), _dev_u64([100])
    _say("device misaligned")
    K.kvcopy_batch_device(ds.data_ptr(), dt.data_ptr(), dz.data_ptr(), dn.data_ptr(), 100, W.D2D,
                          8, base)
    torch.cuda.synchronize()
    assert _status(base) == K.DEVICE_BAD_ALIGN
    assert np.all(res.image(1) == wl.arenas[1].sentinel)
    res.free()


def test_device_empty_count(K):
    from block_copy_amd.harness import Resident
    wl = W.irregular(seed=33, n=50, dir_=W.D2D)
    res = Resident(wl)
    b = wl.batches[0]
    s, d = res.addrs[0]
    ws, base = _workspace(K, 50)
    ds, dt, dz, dn = _dev_u64(s), _dev_u64(d), _dev_u64(b.size), _dev_u64([0])
    _say("device count 0")
    K.kvcopy_batch_device(ds.data_ptr(), dt.data_ptr(), dz.data_ptr(), dn.data_ptr(), 50, W.D2D,
                          8, base)
    torch.cuda.synchronize()
    assert _status(base) == 0
    assert np.all(res.image(1) == wl.arenas[1].sentinel)
    res.free()


def _slot_descs(rng, n, src_len, slot, n_slots, s_base, d_base):
    """n descriptors into distinct destination slots; sizes are 8-byte multiples <= slot."""
    size = (8 * rng.integers(1, slot // 8 + 1, n)).astype(np.uint64)
    slots = rng.choice(n_slots, size=n, replace=False).astype(np.uint64)
    so = (8 * rng.integers(0, (src_len - slot) // 8, n)).astype(np.uint64)
    return s_base + so, d_base + slots * slot, size


def test_device_batch_in_a_hip_graph(K):
    """Captured once; replayed with new descriptor lists and counts written by
    eager copies between replays; every replay checked against the oracle."""
    from block_copy_amd.harness import Resident
    slot, n_slots, max_n = 8192, 1024, 600
    wl = W.Workload("graph", [W.Arena("src", 4 << 20, "device", "random", seed=77),
                              W.Arena("dst", slot * n_slots, "host", "sentinel")], [])
    res = Resident(wl)
    sb, db = res.bases
    ds, dt, dz = (torch.zeros(max_n, dtype=torch.int64, device="cuda") for _ in range(3))
    dn = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws, base = _workspace(K, max_n)
    stream = torch.cuda.Stream()
    rng = np.random.default_rng(5)
    src_img = wl.arenas[0].host_image()
    exp = np.full(slot * n_slots, wl.arenas[1].sentinel, np.uint8)

    def load(n):
        s, d, z = _slot_descs(rng, n, 4 << 20, slot, n_slots, sb, db)
        for t, a in ((ds, s), (dt, d), (dz, z)):
            t[:n].copy_(torch.from_numpy(a.view(np.int64)))
        dn.fill_(n)
        torch.cuda.synchronize()
        oracle.copy(s, d, z, [(sb, src_img)], [(db, exp)])

    _say("graph capture")
    load(10)
    with torch.cuda.stream(stream):   # warm-up launch outside the graph
        K.kvcopy_batch_device(ds.data_ptr(), dt.data_ptr(), dz.data_ptr(), dn.data_ptr(), max_n,
                              W.D2H, 32, base, stream=stream.cuda_stream)
    torch.cuda.synchronize()
    assert_same(res.image(1), exp, "graph warm-up")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        K.kvcopy_batch_device(ds.data_ptr(), dt.data_ptr(), dz.data_ptr(), dn.data_ptr(), max_n,
                              W.D2H, 32, base, stream=stream.cuda_stream)
    torch.cuda.synchronize()
    for rep, n in enumerate((37, 600, 1, 255)):
        _say("graph replay", rep, "n", n)
        load(n)
        g.replay()
        torch.cuda.synchronize()
        assert _status(base) == 0
        assert_same(res.image(1), exp, f"graph replay {rep} (n={n})")
    res.free()
