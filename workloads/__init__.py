"""Seeded synthetic inputs for the batched descriptor copy.

This module is shared by the tests, the smoke check and bench.py: it feeds the
same inputs to the oracle and to the GPU library.  It holds no part of the
method itself (no coalescing, chunking or copying): it only draws descriptor
lists as (arena, offset) pairs and says how each arena is filled.

Workload shapes follow the pages' workloads:
  * PegaFlow issue #408, "Test setup": 16,384 shuffled 4 KiB descriptors per
    direction, 64 MiB H2D + 64 MiB D2H per burst, mapped pinned host payload,
    H2D and D2H on separate streams.
  * vLLM PR #42212 report, "Features and motivation": 4-24 KiB CPU->GPU
    descriptors, real traffic mostly 8-16 KiB.
  * FreeToken issue #751, "Setup": 256 experts per layer in 6 banks, 3,164
    slots, 26-39 missed experts per call.
Where those descriptions leave a choice open, the reading taken is stated on
the generator that makes it.

Arena fills: "random" = uniform random bytes from NumPy's PCG64 seeded with
the arena's seed; "sentinel" = every byte equal to ``sentinel``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

H2D, D2H, D2D = 0, 1, 2
SENTINEL_A = 0xA5
SENTINEL_B = 0x5A
KIB = 1024
MIB = 1024 * 1024


@dataclass
class Arena:
    name: str
    nbytes: int
    where: str            # "device" or "host" (mapped pinned)
    fill: str             # "random" or "sentinel"
    seed: int = 0
    sentinel: int = SENTINEL_A

    def host_image(self) -> np.ndarray:
        """The arena's initial contents as a host uint8 array."""
        if self.fill == "sentinel":
            return np.full(self.nbytes, self.sentinel, dtype=np.uint8)
        rng = np.random.default_rng(self.seed)
        return np.frombuffer(bytearray(rng.bytes(self.nbytes)), dtype=np.uint8)


@dataclass
class Batch:
    """One descriptor list; descriptor i copies size[i] bytes from
    arenas[src_arena[i]] + src_off[i] to arenas[dst_arena[i]] + dst_off[i]."""
    dir: int
    src_arena: np.ndarray   # int32 index into Workload.arenas
    src_off: np.ndarray     # uint64
    dst_arena: np.ndarray
    dst_off: np.ndarray
    size: np.ndarray        # uint64

    @property
    def n(self) -> int:
        return int(self.size.shape[0])

    @property
    def nbytes(self) -> int:
        return int(self.size.sum(dtype=np.uint64))

    def addresses(self, bases):
        """Absolute (src, dst) addresses given the arenas' base addresses."""
        b = np.asarray(bases, dtype=np.uint64)
        return b[self.src_arena] + self.src_off, b[self.dst_arena] + self.dst_off


@dataclass
class Workload:
    name: str
    arenas: list
    batches: list           # submitted concurrently, one stream each
    info: dict = field(default_factory=dict)

    @property
    def nbytes(self) -> int:
        return sum(b.nbytes for b in self.batches)


def _batch(dir_, sa, so, da, do, sz):
    n = len(sz)
    return Batch(dir_,
                 np.full(n, sa, np.int32) if np.isscalar(sa) else np.asarray(sa, np.int32),
                 np.asarray(so, np.uint64),
                 np.full(n, da, np.int32) if np.isscalar(da) else np.asarray(da, np.int32),
                 np.asarray(do, np.uint64),
                 np.asarray(sz, np.uint64))


# ---------------------------------------------------------------------------
# Fixed-size block workloads
# ---------------------------------------------------------------------------

def d2d_blocks(seed=0, n=1024, pool_blocks=4096, block=4 * KIB, sentinel=SENTINEL_A):
    """D2D batch: n blocks gathered/scattered between two device pools.

    Source blocks = first n entries of a seeded permutation of pool A's block
    indices; destination blocks = first n of an independent permutation of
    pool B's.  Pool A is random, pool B is sentinel-filled.
    """
    rng = np.random.default_rng(seed)
    src_blk = rng.permutation(pool_blocks)[:n]
    dst_blk = rng.permutation(pool_blocks)[:n]
    arenas = [Arena("poolA", pool_blocks * block, "device", "random", seed=seed * 1000 + 1),
              Arena("poolB", pool_blocks * block, "device", "sentinel", sentinel=sentinel)]
    b = _batch(D2D, 0, src_blk.astype(np.uint64) * block, 1, dst_blk.astype(np.uint64) * block,
               np.full(n, block, np.uint64))
    return Workload(f"d2d_{n}x{block // KIB}KiB", arenas, [b],
                    {"n": n, "block": block, "pool_blocks": pool_blocks})


def d2d_rotation(seeds=tuple(range(1, 9)), n=65536, pool_blocks=262144, block=4 * KIB,
                 sentinel=SENTINEL_A):
    """Several D2D batches over the same two pools, applied one after another:
    batch k draws its n source and n destination blocks as d2d_blocks(seeds[k])
    does, and the pools are those of d2d_blocks(seeds[0]).  Calls that cycle
    through the batches touch up to len(seeds) times the blocks of one batch,
    so a later call finds little of an earlier call's data in the caches.
    Destinations of different batches may coincide (the batches are
    sequential: a later batch's bytes win)."""
    first = d2d_blocks(seeds[0], n, pool_blocks, block, sentinel)
    batches = [d2d_blocks(sd, n, pool_blocks, block, sentinel).batches[0] for sd in seeds]
    return Workload(f"d2d_rotation_{len(seeds)}x{n}x{block // KIB}KiB", first.arenas, batches,
                    {"n": n, "block": block, "pool_blocks": pool_blocks, "seeds": list(seeds),
                     "sequential": True})


def distinct_calls(seed=0, calls=300, n=8192, block=64, src_blocks=65536, sentinel=SENTINEL_A):
    """`calls` D2D batches of n blocks each, every batch writing its own
    destination blocks: batch i scatters n seeded random source blocks (drawn
    with replacement from a random pool) to a seeded permutation of
    destination blocks [i*n, (i+1)*n).  No two batches touch the same
    destination byte, so every call's result stays visible in the final
    image and a call that ran with another call's worklist shows up."""
    rng = np.random.default_rng(seed)
    arenas = [Arena("src", src_blocks * block, "device", "random", seed=seed * 1000 + 1),
              Arena("dst", calls * n * block, "device", "sentinel", sentinel=sentinel)]
    batches = []
    for i in range(calls):
        src = rng.integers(0, src_blocks, n).astype(np.uint64)
        dst = (np.uint64(i * n) + rng.permutation(n).astype(np.uint64))
        batches.append(_batch(D2D, 0, src * block, 1, dst * block, np.full(n, block, np.uint64)))
    return Workload(f"distinct_{calls}x{n}x{block}B", arenas, batches,
                    {"calls": calls, "n": n, "block": block, "sequential": True})


def kv_blocks(seed=0, directions="both", n=16384, pool_blocks=65536, block=4 * KIB,
              sentinel=SENTINEL_A):
    """H2D and/or D2H batches of n shuffled blocks against a device KV pool.

    Reading of "shuffled descriptors": each host buffer holds n blocks, and
    its block order is a seeded permutation of 0..n-1; the device blocks are a
    seeded sample of distinct indices of the pool.  With both directions the
    H2D destinations and the D2H sources are disjoint samples, and each
    direction has its own host buffer, so the two batches never touch the
    same bytes.

    Arenas: 0 = device pool (random), 1 = host H2D source (random),
    2 = host D2H destination (sentinel).
    """
    if directions not in ("both", "h2d", "d2h"):
        raise ValueError(directions)
    rng = np.random.default_rng(seed)
    need = 2 * n if directions == "both" else n
    if need > pool_blocks:
        raise ValueError("pool too small for the requested blocks")
    dev = rng.permutation(pool_blocks)[:need].astype(np.uint64)
    host_h2d = rng.permutation(n).astype(np.uint64)
    host_d2h = rng.permutation(n).astype(np.uint64)
    arenas = [Arena("kvpool", pool_blocks * block, "device", "random", seed=seed * 1000 + 1),
              Arena("host_h2d_src", n * block, "host", "random", seed=seed * 1000 + 2),
              Arena("host_d2h_dst", n * block, "host", "sentinel", sentinel=sentinel)]
    sz = np.full(n, block, np.uint64)
    batches = []
    if directions in ("both", "h2d"):
        batches.append(_batch(H2D, 1, host_h2d * block, 0, dev[:n] * block, sz))
    if directions in ("both", "d2h"):
        d = dev[n:2 * n] if directions == "both" else dev[:n]
        batches.append(_batch(D2H, 0, d * block, 2, host_d2h * block, sz))
    return Workload(f"kv_{directions}_{n}x{block // KIB}KiB", arenas, batches,
                    {"n": n, "block": block, "pool_blocks": pool_blocks})


# ---------------------------------------------------------------------------
# Mixed sizes with partial adjacency
# ---------------------------------------------------------------------------

def mixed_sizes(rng, n):
    """8 B-multiple sizes: with p = 0.7 uniform over [8 KiB, 16 KiB]; else
    uniform over [4 KiB, 8 KiB) and (16 KiB, 28 KiB].

    Reading: "uniform in 4-28 KiB with 70% in 8-16 KiB" cannot hold as
    written (a uniform law would put a third there), so it is read as this
    mixture.  Its mean is about 13.8 KiB; about half the sizes are odd
    multiples of 8 (not 16 B multiples).
    """
    core = 8192 + 8 * rng.integers(0, 1025, n)                 # 8192 .. 16384
    lo = 4096 + 8 * np.arange(512)                               # 4096 .. 8184
    hi = 16392 + 8 * np.arange(1536)                             # 16392 .. 28672
    side = np.concatenate([lo, hi])[rng.integers(0, 2048, n)]
    return np.where(rng.random(n) < 0.7, core, side).astype(np.uint64)


def _place_runs(rng, run_bytes, gap=64, align=256):
    """Offsets of runs placed in a seeded shuffled order, each run starting
    `align`-aligned and at least `gap` bytes after the previous one."""
    order = rng.permutation(len(run_bytes))
    off = np.zeros(len(run_bytes), np.uint64)
    cur = 0
    for r in order:
        off[r] = cur
        cur = cur + int(run_bytes[r]) + gap
        cur = (cur + align - 1) // align * align
    return off, cur


def h2d_mixed(seed=0, n=4096, adjacent_frac=0.25, sentinel=SENTINEL_A):
    """H2D batch with mixed sizes where a quarter of descriptors continue
    their predecessor in both source and destination.

    Reading of "25% adjacent in both src and dst": exactly floor(0.25 n)
    indices, drawn from 1..n-1, start where descriptor i-1 ends, in both
    arenas.  The resulting runs are placed in independently shuffled orders
    in the host and device arenas, 256 B-aligned with >= 64 B gaps.
    Arenas: 0 = host source (random), 1 = device destination (sentinel).
    """
    rng = np.random.default_rng(seed)
    size = mixed_sizes(rng, n)
    cont = np.zeros(n, bool)
    k = int(adjacent_frac * n)
    if n > 1 and k:
        cont[1 + rng.choice(n - 1, size=k, replace=False)] = True
    run_id = np.cumsum(~cont) - 1                 # run index of each descriptor
    n_runs = int(run_id[-1]) + 1 if n else 0
    run_bytes = np.zeros(n_runs, np.uint64)
    np.add.at(run_bytes, run_id, size)
    # offset of each descriptor inside its run
    ends = np.cumsum(size, dtype=np.uint64)
    starts = ends - size
    run_first = np.zeros(n_runs, np.int64)
    run_first[run_id[~cont]] = np.nonzero(~cont)[0]
    in_run = starts - starts[run_first[run_id]]
    h_off, h_len = _place_runs(rng, run_bytes)
    d_off, d_len = _place_runs(rng, run_bytes)
    arenas = [Arena("host_src", max(h_len, 256), "host", "random", seed=seed * 1000 + 3),
              Arena("dev_dst", max(d_len, 256), "device", "sentinel", sentinel=sentinel)]
    b = _batch(H2D, 0, h_off[run_id] + in_run, 1, d_off[run_id] + in_run, size)
    return Workload(f"h2d_mixed_{n}", arenas, [b],
                    {"n": n, "runs": n_runs, "adjacent": k})


# ---------------------------------------------------------------------------
# MoE expert gather
# ---------------------------------------------------------------------------

MOE_ROWS = (1048576, 65536, 4096, 524288, 32768, 4096)


def moe_arenas(n_experts=256, n_slots=3164, rows=MOE_ROWS, seed=0, sentinel=SENTINEL_A):
    """Host banks b = 0..5, [n_experts, rows[b]] each (random), then device
    slot caches b = 0..5, [n_slots, rows[b]] each (sentinel)."""
    ar = [Arena(f"bank{b}", n_experts * r, "host", "random", seed=seed * 1000 + 10 + b)
          for b, r in enumerate(rows)]
    ar += [Arena(f"cache{b}", n_slots * r, "device", "sentinel", sentinel=sentinel)
           for b, r in enumerate(rows)]
    return ar


def moe_call(rng, n_experts=256, n_slots=3164, rows=MOE_ROWS, misses=(26, 39)):
    """One gather call: m ~ U{misses} experts (distinct) into m distinct slots.

    Reading: every slot counts as free; experts and slots are drawn without
    replacement on every call.  Descriptors are expert-major, bank-minor.
    """
    m = int(rng.integers(misses[0], misses[1] + 1))
    experts = rng.choice(n_experts, size=m, replace=False)
    slots = rng.choice(n_slots, size=m, replace=False)
    nb = len(rows)
    r = np.asarray(rows, np.uint64)
    bank = np.tile(np.arange(nb), m)
    e = np.repeat(experts, nb).astype(np.uint64)
    s = np.repeat(slots, nb).astype(np.uint64)
    return _batch(H2D, bank, e * r[bank], nb + bank, s * r[bank], r[bank])


def moe_gather(seed=0, calls=1, n_experts=256, n_slots=3164, rows=MOE_ROWS, misses=(26, 39),
               sentinel=SENTINEL_A):
    """Expert gather from pinned host banks into the device slot cache.

    Returns a workload whose ``batches`` are successive calls (meant to be run
    one after another on one stream, not concurrently): ``info["sequential"]``.
    """
    rng = np.random.default_rng(seed)
    arenas = moe_arenas(n_experts, n_slots, rows, seed, sentinel)
    batches = [moe_call(rng, n_experts, n_slots, rows, misses) for _ in range(calls)]
    return Workload(f"moe_gather_{calls}calls", arenas, batches,
                    {"sequential": True, "n_experts": n_experts, "n_slots": n_slots,
                     "rows": list(rows)})


# ---------------------------------------------------------------------------
# Small irregular batches for edge cases
# ---------------------------------------------------------------------------

def irregular(seed=0, n=64, max_size=40 * KIB, dir_=D2D, src_where="device", dst_where="device",
              misalign=True, zero_frac=0.0, sentinel=SENTINEL_A, shared_src=False):
    """Random 8 B-aligned descriptors with distinct destinations.

    Sizes are multiples of 8 in [8, max_size].  With ``misalign`` the source
    and destination offsets are independent 8 B multiples, so src and dst
    differ mod 16 for about half the descriptors.  ``zero_frac`` of the
    descriptors get size 0.  With ``shared_src`` several descriptors read
    overlapping source bytes (legal: only destinations must be disjoint).
    """
    rng = np.random.default_rng(seed)
    size = (8 * rng.integers(1, max_size // 8 + 1, n)).astype(np.uint64)
    if zero_frac:
        size[rng.random(n) < zero_frac] = 0

    def place(shared):
        if shared:
            span = int(size.max()) + 4096
            return (8 * rng.integers(0, 512, n)).astype(np.uint64), span + 4096
        order = rng.permutation(n)
        off = np.zeros(n, np.uint64)
        cur = 0
        for i in order:
            cur += 8 * int(rng.integers(0, 9)) if misalign else 0
            if not misalign:
                cur = (cur + 15) // 16 * 16
            off[i] = cur
            cur += int(size[i]) + 8 * int(rng.integers(1, 4))
        return off, cur + 64

    s_off, s_len = place(shared_src)
    d_off, d_len = place(False)
    arenas = [Arena("src", s_len, src_where, "random", seed=seed * 1000 + 5),
              Arena("dst", d_len, dst_where, "sentinel", sentinel=sentinel)]
    b = _batch(dir_, 0, s_off, 1, d_off, size)
    return Workload(f"irregular_{n}", arenas, [b], {"n": n})


# ---------------------------------------------------------------------------
# Randomized batches for stress tests
# ---------------------------------------------------------------------------

def random_batch(seed, max_n=3000):
    """One random descriptor list of every shape the contract allows.

    Direction uniform over H2D / D2H / D2D; n log-uniform in [1, max_n];
    sizes log-uniform over 8-byte multiples from 8 B to 256 KiB, with a
    random fraction of zeros; descriptors come in runs that are adjacent in
    both arenas (so coalescing applies) of random length; runs start at
    independent 8-byte offsets in the two arenas (src and dst differ mod 16
    about half the time), in shuffled order with small gaps.  Destinations
    never overlap; sources do not either.
    """
    rng = np.random.default_rng(seed)
    dir_ = int(rng.integers(0, 3))
    n = max(1, int(round(np.exp(rng.uniform(0, np.log(max_n))))))
    size = (8 * np.exp(rng.uniform(0, np.log(32768), n)).astype(np.int64)).astype(np.uint64)
    size[rng.random(n) < rng.uniform(0, 0.2)] = 0
    cont = rng.random(n) < rng.uniform(0, 0.6)      # descriptor i continues i-1
    cont[0] = False
    starts = np.flatnonzero(~cont)
    runs = [(int(a), int(b)) for a, b in zip(starts, list(starts[1:]) + [n])]

    def place():
        off = np.zeros(n, np.uint64)
        cur = 0
        for r in rng.permutation(len(runs)):
            a, b = runs[r]
            cur += 8 * int(rng.integers(0, 16))
            for i in range(a, b):
                off[i] = cur
                cur += int(size[i])
            cur += 8 * int(rng.integers(1, 8))
        return off, cur + 64

    s_off, s_len = place()
    d_off, d_len = place()
    where = {H2D: ("host", "device"), D2H: ("device", "host"), D2D: ("device", "device")}[dir_]
    arenas = [Arena("src", s_len, where[0], "random", seed=seed * 1000 + 7),
              Arena("dst", d_len, where[1], "sentinel")]
    b = _batch(dir_, 0, s_off, 1, d_off, size)
    return Workload(f"random_{seed}", arenas, [b], {"n": n, "runs": len(runs)})



def combine(name, *wls):
    """One workload holding the arenas and batches of several, in order.

    Each input's arena indices are renumbered past the arenas before it, so
    the batches of different inputs touch disjoint arenas (no overlap across
    them); used to hand two unrelated lists to one call.
    """
    arenas, batches = [], []
    for wl in wls:
        base = len(arenas)
        arenas.extend(wl.arenas)
        for b in wl.batches:
            batches.append(Batch(b.dir, b.src_arena + base, b.src_off.copy(), b.dst_arena + base,
                                 b.dst_off.copy(), b.size.copy()))
    return Workload(name, arenas, batches, {"parts": [wl.name for wl in wls]})
