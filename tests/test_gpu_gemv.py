"""The measurement-only harness kernels: the bf16 GEMV (the synthetic decode
loop of the interference benchmark) against a float32 CPU reference of the
same product, and the scattered read-only and write-only passes that bound
the D2D copy."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def DL():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_copy_amd import decode_load
    return decode_load


def _ref(W, x):
    return W.float().cpu() @ x.float().cpu()


@pytest.mark.parametrize("rows,cols", [(9728, 2560), (2560, 9728), (7, 8), (65, 1032), (1, 4096)])
def test_gemv_matches_fp32_reference(DL, rows, cols):
    print("[case] gemv", rows, cols, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(rows * 7 + cols)
    W = (torch.randn(rows, cols, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    x = torch.randn(cols, generator=g, device="cuda").to(torch.bfloat16)
    y = torch.empty(rows, dtype=torch.bfloat16, device="cuda")
    DL.gemv(W, x, y)
    torch.cuda.synchronize()
    ref = _ref(W, x)
    got = y.float().cpu()
    # bf16 output rounding (half an ulp = 2^-8 relative) plus fp32 summation-order noise
    tol = ref.abs() * 2.0 ** -8 + 1e-5 * ref.abs().max() + 1e-6
    assert torch.all((got - ref).abs() <= tol), float(((got - ref).abs() - tol).max())


def test_chain_runs_products_in_order(DL):
    print("[case] gemv chain", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    shapes = [(96, 64), (64, 96), (96, 64)]
    Ws = [(torch.randn(s, generator=g, device="cuda") * 0.1).to(torch.bfloat16) for s in shapes]
    acts = [torch.randn(64, generator=g, device="cuda").to(torch.bfloat16)]
    acts += [torch.empty(s[0], dtype=torch.bfloat16, device="cuda") for s in shapes]
    DL.Chain(Ws, acts).run()
    torch.cuda.synchronize()
    for i, W in enumerate(Ws):
        ref = _ref(W, acts[i])
        got = acts[i + 1].float().cpu()
        tol = ref.abs() * 2.0 ** -8 + 1e-5 * ref.abs().max() + 1e-6
        assert torch.all((got - ref).abs() <= tol), i


@pytest.mark.parametrize("blk", [4096, 16, 1040, 16384])
def test_scattered_passes_touch_exactly_their_blocks(DL, blk):
    """The D2D ceiling's measurement passes: the write pass fills exactly the
    listed blocks with its pattern and nothing else; the read pass leaves
    memory and its sink untouched."""
    print("[case] scattered passes", blk, flush=True)
    nblk, n = 64, 23
    pool = torch.full((nblk * blk + 64,), 0x11, dtype=torch.uint8, device="cuda")
    g = torch.Generator().manual_seed(blk)
    idx = torch.randperm(nblk, generator=g)[:n]
    addrs = (pool.data_ptr() + idx.to(torch.int64) * blk).to("cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    DL.gather_read(addrs, blk, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    assert torch.all(pool == 0x11)
    DL.scatter_write(addrs, blk, 0xA5A5A5A5)
    torch.cuda.synchronize()
    want = torch.full((nblk * blk + 64,), 0x11, dtype=torch.uint8)
    for i in idx.tolist():
        want[i * blk:(i + 1) * blk] = 0xA5
    assert torch.equal(pool.cpu(), want)


def test_scattered_passes_reject_bad_sizes(DL):
    print("[case] scattered passes: bad sizes", flush=True)
    pool = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    addrs = torch.tensor([pool.data_ptr()], dtype=torch.int64, device="cuda")
    for blk in (0, 8, 20000):
        with pytest.raises(ValueError):
            DL.scatter_write(addrs, blk, 1)
    with pytest.raises(ValueError):
        DL.scatter_write(addrs[:0], 16, 1)


def test_c_caller_latency_tool(DL):
    """kvcopy_latency (kvcopy_batch timed from C, in a child process) runs the
    batches bench.py hands it and finds every destination range equal to its
    source."""
    print("[case] kvcopy_latency", flush=True)
    import bench
    import workloads as W
    rows = bench.c_caller_latency([("d2d_small", W.d2d_blocks(seed=3, n=200, pool_blocks=512), 0),
                                   ("h2d_mixed_16", W.h2d_mixed(seed=1, n=16), -1),
                                   ("d2h_irregular", W.irregular(seed=5, n=300, dir_=W.D2H,
                                                                 src_where="device",
                                                                 dst_where="host"), 8)])
    assert "error" not in rows, rows
    for name in ("d2d_small", "h2d_mixed_16", "d2h_irregular"):
        r = rows[name]
        assert r["ranges_wrong"] == 0 and r["ranges_checked"] == r["descriptors"], r
        assert 0 < r["host_us_p50"] <= r["wall_us_p50"], r
