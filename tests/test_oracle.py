"""Pins for the CPU oracle (oracle/), checked against things other than itself.

* Hand-worked fixtures under tests/golden/ (the pages print no worked example,
  so these are derived by hand from the definition and say so).
* Brute force: a byte-by-byte Python loop over tiny arenas, exhaustive for
  one descriptor and sampled for two and three.
* Special cases: one descriptor is a numpy slice assignment; a run of
  adjacent descriptors is one contiguous slice copy.
* Invariants: destination bytes equal source bytes, bytes outside every
  destination range keep their fill (two different fills), bytes moved equal
  the sum of sizes, sources untouched, order independence, idempotence,
  coalesced input gives the same image.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import plan as oplan
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force(descs, src_arenas, dst_arenas):
    """Byte-by-byte: D[d + x] = S[s + x] for x < size, descriptor by descriptor."""
    out = [img.copy() for _, img in dst_arenas]
    for s, d, n in descs:
        for x in range(n):
            sv = None
            for base, img in src_arenas:
                if base <= s + x < base + len(img):
                    sv = img[s + x - base]
            assert sv is not None
            done = False
            for k, (base, img) in enumerate(dst_arenas):
                if base <= d + x < base + len(img):
                    out[k][d + x - base] = sv
                    done = True
            assert done
    return out


def run_oracle(descs, src_arenas, dst_arenas):
    dsts = [(b, img.copy()) for b, img in dst_arenas]
    a = np.array(descs, dtype=np.uint64).reshape(-1, 3)
    moved = oracle.copy(a[:, 0], a[:, 1], a[:, 2], src_arenas, dsts)
    return [img for _, img in dsts], moved


# --------------------------------------------------------------------------
# Hand-worked fixtures
# --------------------------------------------------------------------------

def test_golden_copy_cases():
    cases = json.load(open(os.path.join(GOLDEN, "copy_cases.json")))["cases"]
    for c in cases:
        src = [(a["base"], ((a["src_fill_base"] + np.arange(a["len"])) % 256).astype(np.uint8))
               for a in c["src_arenas"]]
        dst = [(a["base"], np.full(a["len"], a["dst_fill"], np.uint8)) for a in c["dst_arenas"]]
        out, moved = run_oracle(c["descs"], src, dst)
        assert moved == c["bytes_moved"], c["name"]
        for img, hx in zip(out, c["expect_hex_per_dst_arena"]):
            assert img.tobytes().hex() == hx, c["name"]


# --------------------------------------------------------------------------
# Brute force on tiny arenas
# --------------------------------------------------------------------------

SIZES = (0, 8, 16, 24, 40)
ARENA = 128
SB, DB = 0x10000, 0x30000


def _tiny_arenas(seed):
    rng = np.random.default_rng(seed)
    src = [(SB, rng.integers(0, 256, ARENA, dtype=np.uint8))]
    dst = [(DB, np.full(ARENA, 0xA5, np.uint8))]
    return src, dst


def _positions(size):
    return [o for o in range(0, ARENA - size + 1, 8)]


def _disjoint(descs):
    iv = sorted((d, d + n) for _, d, n in descs if n)
    return all(a[1] <= b[0] for a, b in zip(iv, iv[1:]))


def test_brute_force_exhaustive_one_descriptor():
    src, dst = _tiny_arenas(1)
    count = 0
    for n in SIZES:
        for so in _positions(n):
            for do in _positions(n):
                descs = [(SB + so, DB + do, n)]
                out, moved = run_oracle(descs, src, dst)
                ref = brute_force(descs, src, dst)
                assert np.array_equal(out[0], ref[0])
                assert moved == n
                count += 1
    assert count > 1000


@pytest.mark.parametrize("n", [0, 2, 3])
def test_brute_force_sampled_multi(n):
    rng = np.random.default_rng(100 + n)
    src, dst = _tiny_arenas(2 + n)
    tried = 0
    target = 1 if n == 0 else 1500
    while tried < target:
        descs = []
        for _ in range(n):
            sz = int(rng.choice(SIZES))
            descs.append((SB + int(rng.choice(_positions(sz))),
                          DB + int(rng.choice(_positions(sz))), sz))
        if not _disjoint(descs):
            continue
        out, moved = run_oracle(descs, src, dst)
        ref = brute_force(descs, src, dst)
        assert np.array_equal(out[0], ref[0]), descs
        assert moved == sum(d[2] for d in descs)
        tried += 1


def test_outside_arena_is_reported():
    src, dst = _tiny_arenas(3)
    with pytest.raises(ValueError):
        run_oracle([(SB + ARENA - 8, DB, 16)], src, dst)      # source runs past the arena
    with pytest.raises(ValueError):
        run_oracle([(SB, DB - 8, 8)], src, dst)               # destination before the arena


# --------------------------------------------------------------------------
# Textbook special cases
# --------------------------------------------------------------------------

def test_single_descriptor_is_a_slice_copy():
    rng = np.random.default_rng(7)
    s_img = rng.integers(0, 256, 1 << 16, dtype=np.uint8)
    d_img = np.full(1 << 16, 0x5A, np.uint8)
    for _ in range(50):
        n = 8 * int(rng.integers(0, 2000))
        so = 8 * int(rng.integers(0, ((1 << 16) - n) // 8 + 1))
        do = 8 * int(rng.integers(0, ((1 << 16) - n) // 8 + 1))
        out, moved = run_oracle([(SB + so, DB + do, n)], [(SB, s_img)], [(DB, d_img)])
        ref = d_img.copy()
        ref[do:do + n] = s_img[so:so + n]
        assert np.array_equal(out[0], ref) and moved == n


def test_adjacent_run_is_one_contiguous_copy():
    rng = np.random.default_rng(8)
    s_img = rng.integers(0, 256, 1 << 16, dtype=np.uint8)
    d_img = np.full(1 << 16, 0xA5, np.uint8)
    sizes = 8 * rng.integers(1, 200, 20)
    so, do = 64, 1024
    descs, x = [], 0
    for n in sizes:
        descs.append((SB + so + x, DB + do + x, int(n)))
        x += int(n)
    out, _ = run_oracle(descs, [(SB, s_img)], [(DB, d_img)])
    ref = d_img.copy()
    ref[do:do + x] = s_img[so:so + x]
    assert np.array_equal(out[0], ref)


# --------------------------------------------------------------------------
# Invariants on generated workloads (host images only)
# --------------------------------------------------------------------------

def _images(wl, bases, sentinel=None):
    imgs = []
    for a in wl.arenas:
        if sentinel is not None and a.fill == "sentinel":
            imgs.append(np.full(a.nbytes, sentinel, np.uint8))
        else:
            imgs.append(a.host_image().copy())
    return imgs


def _apply(wl, batch, bases, imgs):
    s, d = batch.addresses(bases)
    src_ids = sorted(set(batch.src_arena.tolist()))
    dst_ids = sorted(set(batch.dst_arena.tolist()))
    src = [(bases[i], imgs[i].copy()) for i in src_ids]     # snapshot before the call
    dst = [(bases[i], imgs[i]) for i in dst_ids]
    return oracle.copy(s, d, batch.size, src, dst)


def _bases(wl):
    # well-separated fake addresses, 4 KiB aligned
    out, cur = [], 1 << 32
    for a in wl.arenas:
        out.append(cur)
        cur += (a.nbytes + (1 << 20)) // 4096 * 4096 + 4096
    return out


@pytest.mark.parametrize("make", [
    lambda: W.irregular(seed=11, n=300, misalign=True),
    lambda: W.irregular(seed=12, n=200, misalign=False, zero_frac=0.1),
    lambda: W.irregular(seed=13, n=100, shared_src=True),
    lambda: W.h2d_mixed(seed=14, n=256),
    lambda: W.d2d_blocks(seed=15, n=64, pool_blocks=256),
])
def test_invariants(make):
    wl = make()
    bases = _bases(wl)
    b = wl.batches[0]
    s_addr, d_addr = b.addresses(bases)
    results = []
    for sentinel in (W.SENTINEL_A, W.SENTINEL_B):
        imgs = _images(wl, bases, sentinel)
        before = [i.copy() for i in imgs]
        moved = _apply(wl, b, bases, imgs)
        assert moved == int(b.size.sum())                                # bytes moved = sum of sizes
        covered = [np.zeros(a.nbytes, bool) for a in wl.arenas]
        for i in range(b.n):
            n = int(b.size[i])
            sa, so = int(b.src_arena[i]), int(b.src_off[i])
            da, do = int(b.dst_arena[i]), int(b.dst_off[i])
            assert np.array_equal(imgs[da][do:do + n], before[sa][so:so + n])   # dst == src
            covered[da][do:do + n] = True
        for k, a in enumerate(wl.arenas):
            if k in set(b.src_arena.tolist()) and k not in set(b.dst_arena.tolist()):
                assert np.array_equal(imgs[k], before[k])                      # sources untouched
            assert np.array_equal(imgs[k][~covered[k]], before[k][~covered[k]])  # outside kept
        results.append(imgs)
        # order independence: a seeded shuffle of the descriptors gives the same image
        perm = np.random.default_rng(5).permutation(b.n)
        imgs2 = [x.copy() for x in before]
        dst_ids = sorted(set(b.dst_arena.tolist()))
        src_ids = sorted(set(b.src_arena.tolist()))
        oracle.copy(s_addr[perm], d_addr[perm], b.size[perm],
                    [(bases[i], before[i].copy()) for i in src_ids],
                    [(bases[i], imgs2[i]) for i in dst_ids])
        for k in dst_ids:
            assert np.array_equal(imgs2[k], imgs[k])
        # idempotence: applying the same batch again changes nothing
        again = [x.copy() for x in imgs]
        oracle.copy(s_addr, d_addr, b.size,
                    [(bases[i], before[i].copy()) for i in src_ids],
                    [(bases[i], again[i]) for i in dst_ids])
        for k in dst_ids:
            assert np.array_equal(again[k], imgs[k])
        # coalesced input gives the same image
        cs, cd, cn = oplan.coalesce(s_addr, d_addr, b.size)
        imgs3 = [x.copy() for x in before]
        oracle.copy(cs, cd, cn, [(bases[i], before[i].copy()) for i in src_ids],
                    [(bases[i], imgs3[i]) for i in dst_ids])
        for k in dst_ids:
            assert np.array_equal(imgs3[k], imgs[k])
    # the two fills differ only outside destination ranges
    for k in sorted(set(b.dst_arena.tolist())):
        if wl.arenas[k].fill == "sentinel":
            assert not np.array_equal(results[0][k], results[1][k]) or b.nbytes == wl.arenas[k].nbytes
