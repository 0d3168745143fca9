"""The seeded generators keep every descriptor inside its arenas and follow the
contract (distinct destinations, no destination overlapping a source), and
produce the shapes the workloads call for.  Checked on the CPU before any of
their descriptors reach the GPU."""
import numpy as np
import pytest

import workloads as W


def _check_contract(wl):
    for b in wl.batches:
        for arena_ids, offs, role in ((b.src_arena, b.src_off, "src"), (b.dst_arena, b.dst_off, "dst")):
            lens = np.array([wl.arenas[i].nbytes for i in arena_ids], np.uint64)
            assert np.all(offs + b.size <= lens), f"{wl.name}: {role} outside its arena"
            assert np.all(offs % 8 == 0) and np.all(b.size % 8 == 0)
        # destinations disjoint within a batch
        key = b.dst_arena.astype(np.uint64) << np.uint64(48) | b.dst_off
        order = np.argsort(key, kind="stable")
        k, z = key[order], b.size[order]
        nz = z > 0
        k, z = k[nz], z[nz]
        assert np.all(k[1:] >= k[:-1] + z[:-1]), f"{wl.name}: overlapping destinations"
        # no destination arena is also a source arena of the same batch
        assert not set(b.src_arena.tolist()) & set(b.dst_arena.tolist())
    if len(wl.batches) > 1 and not wl.info.get("sequential"):
        # concurrent batches: one's destinations never touch another's bytes
        spans = []
        for b in wl.batches:
            spans.append({(int(a), int(o), int(z)) for a, o, z in zip(b.dst_arena, b.dst_off, b.size)})
        for i, b in enumerate(wl.batches):
            for j, other in enumerate(wl.batches):
                if i == j:
                    continue
                mine = {(int(a), int(o)) for a, o in zip(b.src_arena, b.src_off)}
                theirs = {(a, o) for a, o, _ in spans[j]}
                assert not mine & theirs


@pytest.mark.parametrize("make", [
    lambda: W.d2d_blocks(seed=0),
    lambda: W.d2d_blocks(seed=1, n=65536, pool_blocks=262144),
    lambda: W.kv_blocks(seed=0, directions="both"),
    lambda: W.kv_blocks(seed=1, directions="h2d"),
    lambda: W.kv_blocks(seed=1, directions="d2h"),
    lambda: W.h2d_mixed(seed=0, n=16),
    lambda: W.h2d_mixed(seed=0, n=65536),
    lambda: W.moe_gather(seed=0, calls=4),
    lambda: W.moe_gather(seed=4, calls=12, n_experts=32, n_slots=96, misses=(5, 20)),
    lambda: W.irregular(seed=1, n=300),
    lambda: W.irregular(seed=2, n=300, shared_src=True),
    lambda: W.irregular(seed=3, n=300, zero_frac=0.2, misalign=False),
    lambda: W.d2d_rotation(seeds=(1, 2, 3), n=512, pool_blocks=2048),
    lambda: W.combine("pair", W.irregular(seed=4, n=50, dir_=W.H2D, src_where="host"),
                      W.irregular(seed=5, n=9, dir_=W.D2H, dst_where="host")),
])
def test_generators_respect_contract(make):
    _check_contract(make())


def test_shapes():
    wl = W.kv_blocks(seed=0, directions="both")
    assert [b.n for b in wl.batches] == [16384, 16384]
    assert all(b.nbytes == 64 * W.MIB for b in wl.batches)
    assert wl.arenas[0].nbytes == 65536 * 4096
    h2d = wl.batches[0]
    assert sorted((h2d.src_off // 4096).tolist()) == list(range(16384))   # a shuffle of the host buffer
    d = W.d2d_blocks(seed=0)
    assert d.batches[0].n == 1024 and d.batches[0].nbytes == 4 * W.MIB
    assert d.arenas[1].fill == "sentinel" and d.arenas[1].sentinel == 0xA5
    m = W.moe_gather(seed=0, calls=50)
    for b in m.batches:
        assert b.n % 6 == 0 and 26 <= b.n // 6 <= 39
    assert sum(W.MOE_ROWS) == 1679360


def test_mixed_size_distribution():
    rng = np.random.default_rng(0)
    s = W.mixed_sizes(rng, 200000)
    assert s.min() >= 4096 and s.max() <= 28672 and np.all(s % 8 == 0)
    frac_core = np.mean((s >= 8192) & (s <= 16384))
    assert 0.69 < frac_core < 0.72                 # 70 % in 8-16 KiB (the side set never hits it)
    assert 0.45 < np.mean(s % 16 == 8) < 0.55      # about half are not 16 B multiples
    assert 13.5 * 1024 < s.mean() < 14.1 * 1024
    wl = W.h2d_mixed(seed=0, n=4096)
    b = wl.batches[0]
    cont = (b.src_off[1:] == b.src_off[:-1] + b.size[:-1]) & (b.dst_off[1:] == b.dst_off[:-1] + b.size[:-1])
    assert int(cont.sum()) == 1024                 # exactly a quarter continue their predecessor


def test_random_batches_respect_the_contract():
    """Random stress batches: 8-byte aligned, inside their arenas, disjoint
    destinations and sources, and some adjacency for coalescing."""
    merged_somewhere = False
    for seed in range(60):
        wl = W.random_batch(seed)
        b = wl.batches[0]
        assert np.all(b.size % 8 == 0) and np.all(b.src_off % 8 == 0) and np.all(b.dst_off % 8 == 0)
        assert np.all(b.src_off + b.size <= wl.arenas[0].nbytes)
        assert np.all(b.dst_off + b.size <= wl.arenas[1].nbytes)
        for off in (b.dst_off, b.src_off):
            nz = b.size > 0
            o = np.argsort(off[nz], kind="stable")
            lo, hi = off[nz][o], (off + b.size)[nz][o]
            assert np.all(lo[1:] >= hi[:-1])              # no two ranges overlap
        merged_somewhere |= wl.info["runs"] < b.n
    assert merged_somewhere


def test_combine_renumbers_arenas():
    a = W.irregular(seed=4, n=50, dir_=W.H2D, src_where="host")
    b = W.kv_blocks(seed=0, directions="both", n=64, pool_blocks=256)
    c = W.combine("c", a, b)
    assert len(c.arenas) == len(a.arenas) + len(b.arenas)
    assert [x.n for x in c.batches] == [50, 64, 64]
    assert c.batches[0].src_arena.tolist() == a.batches[0].src_arena.tolist()
    k = len(a.arenas)
    for bb, cb in zip(b.batches, c.batches[1:]):
        assert np.array_equal(cb.src_arena, bb.src_arena + k)
        assert np.array_equal(cb.dst_arena, bb.dst_arena + k)
        assert np.array_equal(cb.size, bb.size) and cb.dir == bb.dir
        assert c.arenas[int(cb.dst_arena[0])] is b.arenas[int(bb.dst_arena[0])]


def test_d2d_rotation_shares_pools():
    r = W.d2d_rotation(seeds=(1, 2, 3), n=256, pool_blocks=1024)
    assert len(r.arenas) == 2 and len(r.batches) == 3 and r.info["sequential"]
    for sd, b in zip((1, 2, 3), r.batches):
        one = W.d2d_blocks(sd, 256, 1024).batches[0]
        assert np.array_equal(b.src_off, one.src_off) and np.array_equal(b.dst_off, one.dst_off)
    assert r.arenas[0].seed == W.d2d_blocks(1, 256, 1024).arenas[0].seed
