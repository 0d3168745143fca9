#!/usr/bin/env python3
"""Benchmark of the batched descriptor copy on one MI355X.

Default workload (the headline): bidirectional bursts of 16,384 shuffled
4 KiB descriptors host->device plus 16,384 shuffled 4 KiB descriptors
device->host, submitted concurrently on two streams against a 65,536-block
(256 MiB) device KV pool and mapped pinned host buffers (64 MiB per
direction).  One step = one such burst through the whole path: validate,
coalesce and chunk on the host, one worklist placement and one kernel launch
per direction.  ``value`` is payload bytes moved per second (GB/s = 1e9 B/s)
over the timed steps, inputs resident before the timed region.

Also reported in the same run: each direction alone; the contiguous
hipMemcpyAsync ceilings of the host link (the practical peak); one
hipMemcpyAsync per fragment (the baseline the method replaces); the D2D
gather of 1,024 x 4 KiB blocks and a scaled D2D variant against HBM; and the
CPU oracle timed on the host cores on a bounded sample.  Every GPU result is
checked bit-exact against the oracle images of that leg before the line is
printed.

Other workloads (``--workload``), one JSON line each:
  pair          the headline burst as one kvcopy_batch_pair call (one launch)
  d2d           1,024 x 4 KiB D2D gather (and 65,536 x 4 KiB) against HBM
  mixed         H2D with mixed 4-28 KiB sizes, N = 16, 256, 4,096, 65,536
  moe           MoE expert gather, 100 seeded calls of 26-39 experts x 6 banks
  interference  decode-loop step times while bidirectional bursts run every 50 ms

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--max-wgs G] [--workload X]
Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import hashlib
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s for batched 4–16 KiB descriptor copies (H2D/D2H/D2D), % of link/HBM peak"
PCIE_PEAK_GBS = 64.0      # PCIe 5.0 x16, per direction (MI355X host interface)
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
# Workgroup cap per stream of the headline.  Measured on MI355X with the
# headline burst on streams over disjoint CU halves (Ctx.headline_streams),
# two processes per cap: 8 -> 96.4-97.2 GB/s, 12-32 -> 69-87, 48 -> 96.3,
# 64 -> 96.7-96.8, 96 -> 96.7-97.1, 128 -> 90.6-90.9, 256 -> 85.7-86.3.
# 64 sits inside the broad plateau; the peak at 8 is a narrow one (7 or 9
# workgroups per stream on streams over every CU: 84-90 GB/s).
DEFAULT_MAX_WGS = 64
# Workgroup cap of the one-direction legs (mixed sizes): the library's
# default grid for H2D and D2H.
ONE_WAY_MAX_WGS = 128
REC_BYTES = 24            # one worklist record per chunk
LINK_SETTLE_STEPS = 700   # untimed headline steps (about 1 s) before any host-link figure,
LINK_SETTLE_SECONDS = 1.5  # or this long, whichever ends first (small caps run slow steps)
DIR_NAMES = ("h2d", "d2h", "d2d")
COUNTERS_KV = os.path.join(ROOT, "profiles", "counters_kv_bidirectional.json")
COUNTERS_D2D = os.path.join(ROOT, "profiles", "counters_d2d_blocks.json")
COUNTERS_PAIR = os.path.join(ROOT, "profiles", "counters_kv_pair.json")
KERNEL_SOURCES = [os.path.join(ROOT, "block_copy_amd", "csrc", f)
                  for f in ("kvcopy_kernel.hip", "copy_chunk.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gbs(nbytes, seconds):
    return nbytes / seconds / 1e9


def pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    k = min(len(xs) - 1, max(0, int(round(q / 100.0 * (len(xs) - 1)))))
    return xs[k]


@contextlib.contextmanager
def no_gc():
    """Timed regions run with Python's cyclic garbage collector paused: a
    full collection in a process that holds torch takes tens of milliseconds
    and would land inside whichever call happens to trigger it."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, path=COUNTERS_KV, alg_fetch=None, alg_write=None):
    """Bytes per launch of `kernel` from the committed PMC summary, or None if
    there is none or the kernel source changed since it was taken.  With the
    algorithmic bytes each side must move (fetch: payload reads plus the
    worklist records; write: payload writes), also each side's ratio of
    measured to algorithmic bytes (1.0 = no re-reads, no extra writes)."""
    try:
        with open(path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != kernel_source_hash():
        return None
    k = c.get("kernels", {}).get(kernel)
    if not k:
        return None
    f, w = k["fetch_bytes_per_dispatch_scaled"], k["write_bytes_per_dispatch_scaled"]
    out = {"bytes": f + w, "fetch_bytes": f, "write_bytes": w,
           "source": os.path.relpath(path, ROOT)}
    if alg_fetch and alg_write:
        out.update({"algorithmic_fetch_bytes": int(alg_fetch), "algorithmic_write_bytes": int(alg_write),
                    "fetch_ratio": round(f / alg_fetch, 4), "write_ratio": round(w / alg_write, 4)})
    return out


class Ctx:
    """GPU handles shared by the workloads."""

    def __init__(self, args):
        import numpy as np
        import torch

        import workloads as W
        from block_copy_amd import hiprt
        from block_copy_amd import kvcopy as K
        from block_copy_amd.harness import Resident
        self.np, self.torch, self.W, self.hiprt, self.K, self.Resident = np, torch, W, hiprt, K, Resident
        self.args = args
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        p = torch.cuda.get_device_properties(self.dev)
        log(f"device: {p.name} ({p.gcnArchName}), {p.multi_processor_count} CUs")
        # the two copy streams get a hardware queue each (hiprt.QueueStreams):
        # plain streams may share one and then run the two directions in turn
        self.ncu = p.multi_processor_count
        self._halves = None
        self.stream_kind = "a hardware queue each (full CU mask)"
        try:
            self.queues = hiprt.QueueStreams(2, self.ncu)
            self.sA, self.sB = self.queues.streams
        except RuntimeError as e:
            log(f"  dedicated-queue streams unavailable ({e}); using torch streams")
            self.stream_kind = "torch streams (dedicated queues unavailable)"
            self.sA, self.sB = torch.cuda.Stream(), torch.cuda.Stream()

    def headline_streams(self):
        """The two copy streams of the headline step and their description.
        With --copy-cus halves (the default) each has a hardware queue of its
        own on one half of the CU mask bits, [0, n/2) and [n/2, n): every XCD
        keeps CUs for both (bit i is a CU of XCD i % 8).  Measured on MI355X
        with the headline burst: 96.3-97.1 GB/s at 48-96 workgroups per
        stream against 94.5-95.8 at 64 on streams over every CU.  With
        --copy-cus all they are sA and sB."""
        if self.args.copy_cus != "halves" or getattr(self, "queues", None) is None:
            return self.sA, self.sB, self.stream_kind
        if self._halves is None:
            n = self.ncu
            self._halves = self.hiprt.QueueStreams(2, n, [range(n // 2), range(n // 2, n)])
        n = self.ncu
        return (*self._halves.streams,
                f"a hardware queue each; H2D on CU mask bits 0-{n // 2 - 1}, D2H on "
                f"{n // 2}-{n - 1} (every XCD keeps CUs for both)")

    def close(self):
        """Explicit teardown before the interpreter exits: wait for the GPU,
        destroy the streams made here, and collect the objects (events,
        host buffers) whose finalisers make HIP calls while the runtime is
        still whole (during interpreter shutdown those finalisers skip their
        HIP calls)."""
        self.torch.cuda.synchronize()
        for q in ("queues", "_halves"):
            if getattr(self, q, None) is not None:
                getattr(self, q).destroy()
                setattr(self, q, None)
        gc.collect()
        self.torch.cuda.synchronize()

    def run_steps(self, r, batch_ids, streams, k, max_wgs, events=None, joined=False, **kw):
        """k steps; a step submits each batch on its stream.  With `joined`,
        every stream waits for the others' batches of the step before its
        next one, so the batches of a step start together and the step ends
        when the last one does."""
        if self.args.desc_upload:
            kw["flags"] = kw.get("flags", 0) | self.K.F_DESC_UPLOAD
        if getattr(self.args, "flags", 0):
            kw["flags"] = kw.get("flags", 0) | self.args.flags
        forms = store_forms(self.args.store)
        marks = None
        # profiler runs (--no-events) make no event calls at all (rocprofv3 7.2
        # aborted in its own tool on them): there the host joins the steps
        if joined and len(streams) > 1 and not self.args.no_events:
            marks = [self.hiprt.Event(timing=False) for _ in streams]
        for i in range(k):
            for j, (bi, st) in enumerate(zip(batch_ids, streams)):
                extra = dict(kw)
                if events is not None:
                    extra.update(kernel_begin=events[i][j][0].h, kernel_end=events[i][j][1].h)
                g = max_wgs[j] if isinstance(max_wgs, (list, tuple)) else max_wgs
                form = forms.get(r.wl.batches[bi].dir)
                if form:
                    extra["flags"] = extra.get("flags", 0) | (
                        self.K.F_STORE_SC1 if form == "sc1" else self.K.F_STORE_NT)
                r.submit(bi, g, st, **extra)
            if marks:
                for m, st in zip(marks, streams):
                    m.record(st)
                for j, st in enumerate(streams):
                    for jj, m in enumerate(marks):
                        if jj != j:
                            self.hiprt.stream_wait(st, m)
            elif joined and len(streams) > 1:
                # profiler runs (no event calls): the host waits for both
                # streams, so the next step's kernels again start together
                for st in streams:
                    self.hiprt.stream_sync(st)

    def timed(self, r, batch_ids, streams, k, w, max_wgs, with_events=True, **kw):
        """Seconds per step over k timed steps (after w warm-up steps), and the
        mean kernel-only duration (ms) of each batch from HIP events recorded on
        the stream each kernel runs on."""
        torch = self.torch
        with_events = with_events and not self.args.no_events
        self.run_steps(r, batch_ids, streams, w, max_wgs, **kw)
        torch.cuda.synchronize()
        evs = [[(self.hiprt.Event(), self.hiprt.Event()) for _ in batch_ids] for _ in range(k)] \
            if with_events else None
        with no_gc():
            t0 = time.perf_counter()
            self.run_steps(r, batch_ids, streams, k, max_wgs, evs, **kw)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        if evs:
            kern = [statistics.mean(evs[i][j][0].elapsed_ms(evs[i][j][1]) for i in range(k))
                    for j in range(len(batch_ids))]
        else:   # profiler runs: no events; the step time stands in for the kernel time
            kern = [(t1 - t0) / k * 1e3] * len(batch_ids)
        return (t1 - t0) / k, kern

    def timed_bracketed(self, r, batch_ids, streams, k, w, max_wgs, **kw):
        """Seconds per step over k timed steps, and each stream's mean kernel
        duration (ms): one HIP event pair per stream brackets its k kernels,
        which run back to back (joined=True: step by step), so no timing
        event sits between two kernels."""
        torch, hiprt = self.torch, self.hiprt
        self.run_steps(r, batch_ids, streams, w, max_wgs, **kw)
        torch.cuda.synchronize()
        use_ev = not self.args.no_events
        evs = [(hiprt.Event(), hiprt.Event()) for _ in batch_ids] if use_ev else None
        with no_gc():
            t0 = time.perf_counter()
            if use_ev:
                for (e0, _), st in zip(evs, streams):
                    e0.record(st)
            self.run_steps(r, batch_ids, streams, k, max_wgs, **kw)
            if use_ev:
                for (_, e1), st in zip(evs, streams):
                    e1.record(st)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        if use_ev:
            kern = [e0.elapsed_ms(e1) / k for e0, e1 in evs]
        else:
            kern = [(t1 - t0) / k * 1e3] * len(batch_ids)
        return (t1 - t0) / k, kern

    def pair_step(self, r, stream, max_wgs):
        """One kvcopy_batch_pair call: batch 0 and batch 1 in one launch."""
        (s0, d0), (s1, d1) = r.addrs[0], r.addrs[1]
        self.K.kvcopy_batch_pair(s0, d0, r.wl.batches[0].size, s1, d1, r.wl.batches[1].size,
                                 max_wgs, stream.cuda_stream)

    def latency(self, r, bi, max_wgs, k=100, w=10, **kw):
        """Per-call latency of isolated calls: host time inside kvcopy_batch,
        GPU time from an event recorded before the call to one after it, and
        the synchronous wall time of call + stream sync."""
        hiprt, st = self.hiprt, self.sA
        if self.args.no_events:
            return None
        if self.args.desc_upload:
            kw["flags"] = kw.get("flags", 0) | self.K.F_DESC_UPLOAD
        for _ in range(w):
            r.submit(bi, max_wgs, st, **kw)
        hiprt.stream_sync(st)
        host, gpu, wall = [], [], []
        evs = [(hiprt.Event(), hiprt.Event()) for _ in range(k)]
        with no_gc():
            for e0, e1 in evs:
                t0 = time.perf_counter()
                e0.record(st)
                t1 = time.perf_counter()
                r.submit(bi, max_wgs, st, **kw)
                t2 = time.perf_counter()
                e1.record(st)
                hiprt.stream_sync(st)
                t3 = time.perf_counter()
                host.append((t2 - t1) * 1e6)
                wall.append((t3 - t0) * 1e6)
        gpu = [e0.elapsed_ms(e1) * 1e3 for e0, e1 in evs]
        rd = lambda x: round(x, 2)  # noqa: E731
        return {"host_us_p50": rd(pct(host, 50)), "gpu_us_p50": rd(pct(gpu, 50)),
                "gpu_us_p99": rd(pct(gpu, 99)), "wall_us_p50": rd(pct(wall, 50)),
                "wall_us_p99": rd(pct(wall, 99))}

    def oracle_images(self, wl, r, batch_ids):
        """Host images after applying the batches with the oracle (arena index -> image)."""
        import oracle
        np = self.np
        touched = set()
        for k in batch_ids:
            b = wl.batches[k]
            touched |= set(b.src_arena.tolist()) | set(b.dst_arena.tolist())
        imgs = {i: (wl.arenas[i].host_image().copy() if wl.arenas[i].fill == "random"
                    else np.full(wl.arenas[i].nbytes, wl.arenas[i].sentinel, np.uint8))
                for i in touched}
        for k in batch_ids:
            b = wl.batches[k]
            s, d = r.addrs[k]
            src_ids = sorted(set(b.src_arena.tolist()))
            dst_ids = sorted(set(b.dst_arena.tolist()))
            snap = {i: imgs[i].copy() for i in src_ids}
            oracle.copy(s, d, b.size, [(r.bases[i], snap[i]) for i in src_ids],
                        [(r.bases[i], imgs[i]) for i in dst_ids])
        return imgs

    def verify(self, wl, r, batch_ids, what):
        """Bit-exact check of every destination arena against the oracle; exits on mismatch."""
        np = self.np
        exp = self.oracle_images(wl, r, batch_ids)
        dsts = set()
        for k in batch_ids:
            dsts |= set(wl.batches[k].dst_arena.tolist())
        for i in sorted(dsts):
            got = r.image(i)
            if not np.array_equal(got, exp[i]):
                bad = int(np.flatnonzero(got != exp[i])[0])
                log(f"PARITY FAILURE ({what}) in arena {wl.arenas[i].name} at byte {bad}")
                sys.exit(3)


def parse_wgs(text):
    """--max-wgs: one cap, or "H2D,D2H" (two caps, headline only)."""
    vals = [int(x) for x in text.split(",")]
    if len(vals) == 1:
        return vals[0]
    if len(vals) != 2:
        raise argparse.ArgumentTypeError("expected N or H2D,D2H")
    return vals


def pcie_link():
    """The GPU's negotiated PCIe link as sysfs reports it ({"speed": "32.0 GT/s
    PCIe", "width": 16} for PCIe 5.0 x16), or None when it cannot be read or
    more than one AMD GPU is visible (the card would be ambiguous)."""
    import glob
    found = []
    for d in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(d, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
            with open(os.path.join(d, "current_link_speed")) as f:
                speed = f.read().strip()
            with open(os.path.join(d, "current_link_width")) as f:
                width = int(f.read().strip())
        except (OSError, ValueError):
            continue
        found.append({"speed": speed, "width": width})
    return found[0] if len(found) == 1 else None


def kernel_name(dir_, spec="auto"):
    """The per-chunk copy kernel's symbol for a direction under --store
    (the library stores D2H in the sc1 form on grids of three or more
    workgroups, as every leg that names a kernel runs, and the rest nt)."""
    form = store_forms(spec).get(dir_) or ("sc1" if dir_ == 1 else "nt")
    return f"kvcopy_{DIR_NAMES[dir_]}{'_sc1' if form == 'sc1' else ''}_kernel"


def store_forms(spec):
    """Direction (0 H2D, 1 D2H, 2 D2D) -> "sc1" or "nt" from --store: "auto"
    (the library's choice for every direction), "sc1" or "nt" (every
    direction), or per direction as "h2d:sc1,d2h:nt"."""
    if spec == "auto":
        return {}
    if spec in ("sc1", "nt"):
        return {0: spec, 1: spec, 2: spec}
    out = {}
    for part in spec.split(","):
        d, _, f = part.partition(":")
        if d not in ("h2d", "d2h", "d2d") or f not in ("sc1", "nt", "auto"):
            raise ValueError(f"bad --store part {part!r}")
        if f != "auto":
            out[("h2d", "d2h", "d2d").index(d)] = f
    return out


def base_line(args, value, unit, step_s, config, dtype="u8", higher=True):
    return {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": higher,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "config": config}


# ---------------------------------------------------------------------------
# Headline: bidirectional KV block bursts
# ---------------------------------------------------------------------------

def bench_kv(c: Ctx, args):
    np, torch, W, K, hiprt = c.np, c.torch, c.W, c.K, c.hiprt
    wl = W.kv_blocks(seed=0, directions="both")
    res = c.Resident(wl)
    sA, sB = c.sA, c.sB
    hA, hB, stream_kind = c.headline_streams()     # the headline step's two streams
    step_bytes = wl.nbytes
    n_desc = sum(b.n for b in wl.batches)
    max_wgs = args.max_wgs if args.max_wgs is not None else DEFAULT_MAX_WGS

    def cap_of(j):     # direction j's cap (--max-wgs H2D,D2H gives one per direction)
        return max_wgs[j] if isinstance(max_wgs, list) else max_wgs

    extras = {}
    # Before any figure is taken, the headline's own step runs untimed for
    # about a second (LINK_SETTLE_STEPS).  Measured on MI355X, the start of a
    # process can find the host link slow for a second or so, for the
    # runtime's contiguous copies as much as for the kernel: in one process
    # of nine the contiguous pair read 87.8 GB/s (96.4-96.7 in the others),
    # each direction alone 54 GB/s and the 20-step headline 85.1, while the
    # 30 windows that followed it read 96.5 at the median.  Settling first
    # puts the ceilings, the per-direction legs and the headline on the same
    # steady link.  The headline then takes its own --warmup steps as asked.
    t_settle, done = time.perf_counter(), 0
    while done < LINK_SETTLE_STEPS and time.perf_counter() - t_settle < LINK_SETTLE_SECONDS:
        c.run_steps(res, [0, 1], [hA, hB], 50, max_wgs, joined=True)
        for st in (hA, hB):
            hiprt.stream_sync(st)
        done += 50
    # The host link's contiguous ceilings (DMA, no copy kernel) and, in the
    # full run, each direction alone come next: they are part of the report,
    # and they keep the link in steady use before the headline's own warm-up
    # (measured on MI355X, bidirectional traffic in the first quarter second
    # of a process runs at 51-69 GB/s).
    extras["contiguous_memcpy_ceiling_GBps"] = ceilings(c)
    log(f"  contiguous ceilings: {extras['contiguous_memcpy_ceiling_GBps']}")
    if not args.skip_extras:
        alone = {}
        for j, name in ((0, "h2d"), (1, "d2h")):
            s, _ = c.timed_bracketed(res, [j], [sA], args.steps, args.leg_warmup, cap_of(j))
            _, km = c.timed(res, [j], [sA], args.steps, 2, cap_of(j))
            alone[name] = {"GBps": round(gbs(wl.batches[j].nbytes, s), 3),
                           "ms_per_call": round(s * 1e3, 4), "kernel_ms": round(km[0], 4),
                           "latency": c.latency(res, j, cap_of(j), k=50, w=5)}
            log(f"  {name} alone: {alone[name]}")
        extras["per_direction_alone"] = alone
    log(f"headline: {n_desc} descriptors, {step_bytes} B per step, max_wgs={max_wgs}")
    # No HIP event sits between two kernels (events recorded between the
    # kernels perturb how the two streams overlap): one event pair per stream
    # brackets that stream's back-to-back kernels over the timed steps.
    # The step starts both directions together and ends when both are done
    # (joined): free-running streams drift out of phase over hundreds of
    # steps and leave stretches with one direction running alone.
    step_s, kern_ms = c.timed_bracketed(res, [0, 1], [hA, hB], args.steps, args.warmup, max_wgs,
                                        joined=True)
    value = gbs(step_bytes, step_s)
    log(f"  bidirectional: {step_s * 1e3:.3f} ms/step, {value:.2f} GB/s; mean kernel ms per "
        f"stream {kern_ms}")
    plans = [K.kvcopy_plan(*res.addrs[j], wl.batches[j].size) for j in range(2)]
    algo = [wl.batches[j].nbytes + plans[j].n_chunks * REC_BYTES for j in range(2)]
    ach = [gbs(algo[j], kern_ms[j] / 1e3) for j in range(2)]

    if args.sweep:
        # each direction alone on one stream, and both on the headline's two
        # streams with the steps joined, each point timed as the headline is
        # (one event pair per stream around its back-to-back kernels)
        sweep = {}
        for name, ids, sts in (("h2d", [0], [sA]), ("d2h", [1], [sA]), ("both", [0, 1], [hA, hB])):
            for g in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 0):
                s_, km = c.timed_bracketed(res, ids, sts, max(3, args.steps // 2), args.leg_warmup,
                                           g, joined=len(ids) > 1)
                nbytes = sum(wl.batches[i].nbytes for i in ids)
                sweep[f"{name}/{g}"] = round(gbs(nbytes, s_), 2)
                log(f"  sweep {name} max_wgs={g}: {gbs(nbytes, s_):.2f} GB/s")
        extras["max_wgs_sweep_GBps"] = sweep
    if not args.skip_extras and not args.no_events:
        extras["headline_windows"] = headline_windows(c, res, max_wgs, streams=(hA, hB))
        log(f"  headline windows: {dict((k, v) for k, v in extras['headline_windows'].items() if k not in ('GBps', 'kernel_ms_per_stream'))}")
    if not args.skip_extras:
        alone = extras["per_direction_alone"]
        # a lone D2H list through kvcopy_batch_pair (whose kernel stores in
        # the sc1 form, as kvcopy_batch's D2H kernel does on such grids)
        e_ = np.zeros(0, np.uint64)
        s1_, d1_ = res.addrs[1]
        for _ in range(args.leg_warmup):
            K.kvcopy_batch_pair(s1_, d1_, wl.batches[1].size, e_, e_, e_, K.WGS_AUTO, sA.cuda_stream)
        torch.cuda.synchronize()
        ev0, ev1 = hiprt.Event(), hiprt.Event()
        ev0.record(sA)
        for _ in range(args.steps):
            K.kvcopy_batch_pair(s1_, d1_, wl.batches[1].size, e_, e_, e_, K.WGS_AUTO, sA.cuda_stream)
        ev1.record(sA)
        ms_ = ev0.elapsed_ms(ev1) / args.steps
        alone["d2h_one_list_through_pair"] = {"GBps": round(gbs(wl.batches[1].nbytes, ms_ / 1e3), 3),
                                              "kernel_ms": round(ms_, 4)}
        log(f"  d2h alone through kvcopy_batch_pair: {alone['d2h_one_list_through_pair']}")
        cl = c_caller_latency([(f"kv_{nm}_16384x4KiB", W.kv_blocks(seed=0, directions=nm), cap_of(j))
                               for j, nm in enumerate(("h2d", "d2h"))])
        for nm in ("h2d", "d2h"):
            alone[nm]["latency_c_caller"] = cl.get(f"kv_{nm}_16384x4KiB", cl.get("error"))
        log(f"  each direction alone, C caller: {cl}")
        # the startup probe's choice, and the headline step at that cap
        cap, rates = K.kvcopy_autotune(K.H2D, hA.cuda_stream, hB.cuda_stream)
        auto = {"h2d_d2h": cap, "probe_GBps": {str(k): round(v, 2) for k, v in rates.items()}}
        s_, km = c.timed_bracketed(res, [0, 1], [hA, hB], args.steps, args.leg_warmup, K.WGS_AUTO,
                                   joined=True)
        auto["bidirectional_GBps_at_auto"] = round(gbs(step_bytes, s_), 3)
        if not args.no_events:
            auto["windows_at_auto"] = headline_windows(c, res, K.WGS_AUTO, n=10, streams=(hA, hB))
            auto["windows_at_auto"].pop("kernel_ms_per_stream")
        extras["autotune"] = auto
        log(f"  autotune: {auto}")
        frag = {}
        for j, name, kind in ((0, "h2d", hiprt.H2D_KIND), (1, "d2h", hiprt.D2H_KIND)):
            frag[name] = dma_baselines(c, plans[j], wl.batches[j].nbytes, kind)
            log(f"  DMA baselines {name}: {frag[name]}")
        extras["dma_baselines"] = frag
        extras["dma_baselines_rocm_runtime"] = dma_runtime_baselines()
        extras["one_launch_pair"] = pair_rates(c, res, args)

    if args.counter_calibration:
        counter_calibration(c)

    # verification + cpu_baseline (the oracle on host images of the same step).
    # The DMA baselines above wrote the same destination arenas, so refill
    # them and run one more kernel step before reading the images back.
    res.fill()
    c.run_steps(res, [0, 1], [hA, hB], 1, max_wgs)
    torch.cuda.synchronize()
    final = {i: res.image(i) for i in (0, 2)}        # device pool, host D2H destination
    imgs, cpu = kv_oracle(c, wl, res, args)
    check_kv_images(wl, final, imgs, "")
    if not args.skip_extras:
        # the one-launch call on the same inputs must leave the same images
        res.fill()
        c.pair_step(res, sA, K.WGS_AUTO)
        torch.cuda.synchronize()
        check_kv_images(wl, {i: res.image(i) for i in (0, 2)}, imgs, " (one-launch pair)")
        extras["one_launch_pair"]["parity"] = "bit-exact vs oracle"
    log("  parity: bit-exact against the oracle")
    res.free()

    if not args.skip_extras:
        ceil_h2d = extras["contiguous_memcpy_ceiling_GBps"]["h2d"]
        extras["mixed_h2d"] = mixed_compact(c, args, ceil_h2d)
        extras["moe_gather"] = moe_compact(c, args, ceil_h2d)
        extras["d2d"] = d2d_results(c, args)

    dom = 0 if kern_ms[0] >= kern_ms[1] else 1
    meas_ceil = extras.get("contiguous_memcpy_ceiling_GBps", {}).get(("h2d", "d2h")[dom])
    line = base_line(args, round(value, 3), "GB/s", step_s, {
        "workload": "bidirectional KV block burst: 16,384 shuffled 4 KiB H2D + 16,384 shuffled "
                    "4 KiB D2H per step, concurrent on two streams, 65,536-block device pool, "
                    "mapped pinned host buffers",
        "descriptors_per_step": n_desc, "bytes_per_step": step_bytes,
        "max_wgs": max_wgs, "chunk_bytes": K.CHUNK_DEFAULT, "seed": 0,
        "streams": stream_kind, "store_form": args.store})
    line["roofline"] = {
        "bound": "pcie", "kernel": kernel_name(dom, args.store), "achieved": round(ach[dom], 3),
        "peak": PCIE_PEAK_GBS, "unit": "GB/s", "frac": round(ach[dom] / PCIE_PEAK_GBS, 4),
        "traffic": measured_traffic(kernel_name(dom, args.store), COUNTERS_KV, algo[dom],
                                    wl.batches[dom].nbytes),
        "kernel_ms": round(kern_ms[dom], 4), "algorithmic_bytes_per_launch": algo[dom],
        "measured_ceiling": meas_ceil,
        "frac_of_measured_ceiling": round(ach[dom] / meas_ceil, 4) if meas_ceil else None,
        "other_kernel": {"kernel": kernel_name(1 - dom, args.store),
                         "achieved": round(ach[1 - dom], 3),
                         "kernel_ms": round(kern_ms[1 - dom], 4)},
        "link": pcie_link()}
    # the step against the link's measured two-direction ceiling: contiguous
    # hipMemcpyAsync H2D and D2H of 64 MiB each, concurrent on two streams
    both_ceil = extras.get("contiguous_memcpy_ceiling_GBps", {}).get("both")
    if both_ceil:
        line["roofline"]["measured_ceiling_both_directions"] = both_ceil
        line["roofline"]["frac_step_of_ceiling_both_directions"] = round(value / both_ceil, 4)
    line["cpu_baseline"] = cpu_baseline_record(
        cpu, "whole steps of 16,384 H2D + 16,384 D2H descriptors of 4 KiB")
    line["parity"] = "bit-exact vs oracle"
    line.update(extras)
    return line


def kv_oracle(c: Ctx, wl, res, args):
    """The oracle's images of one bidirectional step (arena index -> uint8
    array), and the oracle timed over whole steps on one host thread and on
    every CPU this process may use (host_cpus)."""
    np = c.np
    import oracle
    imgs = [a.host_image().copy() if a.fill == "random" else np.full(a.nbytes, a.sentinel, np.uint8)
            for a in wl.arenas]
    src_snap = {0: imgs[0].copy(), 1: imgs[1]}
    parts = []
    for j in range(2):
        b = wl.batches[j]
        s, d = res.addrs[j]
        si, di = int(b.src_arena[0]), int(b.dst_arena[0])
        parts.append((s, d, b.size, [(res.bases[si], src_snap[si])], [(res.bases[di], imgs[di])]))
    for p in parts:                                   # the images of one step
        oracle.copy(*p)
    cpus = host_cpus()
    one = oracle_rate(parts, 1, args.cpu_seconds / 2)
    many = oracle_rate(parts, cpus["threads"], args.cpu_seconds / 2)
    log(f"  cpu oracle: 1 thread {one['GBps']:.2f} GB/s, {cpus['threads']} threads "
        f"{many['GBps']:.2f} GB/s ({cpus})")
    return imgs, {"one": one, "many": many, "cpus": cpus}


def host_cpus() -> dict:
    """The CPUs this process may use: os.cpu_count() (nproc), the affinity
    mask, and the cgroup CPU quota (cpu.max, in CPUs) if one is set; the
    oracle's thread count is the smaller of the last two."""
    nproc = os.cpu_count() or 1
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = nproc
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
            if q != "max":
                quota = int(q) / int(per)
    except (OSError, ValueError):
        pass
    threads = aff if quota is None else max(1, min(aff, int(quota)))
    return {"nproc": nproc, "affinity_cpus": aff, "cgroup_cpu_quota": quota, "threads": threads}


def oracle_rate(parts, threads, seconds, trials=5):
    """GB/s of the oracle over whole steps (`parts`: the oracle.copy argument
    tuples of one step) on `threads` host threads.  Each thread copies a
    contiguous, byte-balanced share of every part's descriptors, so the
    threads write disjoint bytes; the oracle releases the interpreter lock
    while it copies.  Median of `trials` timed runs of about seconds/trials
    each."""
    import oracle
    np = sys.modules["numpy"]
    shares = [[] for _ in range(threads)]
    total = 0
    for s, d, z, sa, da in parts:
        z = np.ascontiguousarray(z, dtype=np.uint64)
        cum = np.cumsum(z, dtype=np.uint64)
        total += int(cum[-1]) if len(cum) else 0
        cuts = [0] + [int(np.searchsorted(cum, int(cum[-1]) * k // threads, side="right"))
                      for k in range(1, threads)] + [len(z)]
        for t in range(threads):
            a, b = cuts[t], cuts[t + 1]
            if b > a:
                shares[t].append((np.ascontiguousarray(s[a:b]), np.ascontiguousarray(d[a:b]),
                                  z[a:b].copy(), sa, da))

    def run(reps):
        gate = threading.Barrier(threads + 1)

        def work(t):
            gate.wait()
            for _ in range(reps):
                for args_ in shares[t]:
                    oracle.copy(*args_)
        ths = [threading.Thread(target=work, args=(t,)) for t in range(threads)]
        for th in ths:
            th.start()
        gate.wait()
        t0 = time.perf_counter()
        for th in ths:
            th.join()
        return time.perf_counter() - t0

    t1 = run(1)
    reps = max(1, int(seconds / trials / max(t1, 1e-6)))
    times = [run(reps) for _ in range(trials)]
    dt = statistics.median(times)
    return {"GBps": gbs(total * reps, dt), "reps_per_trial": reps, "trials": trials,
            "threads": threads, "seconds": round(sum(times) + t1, 2)}


def cpu_baseline_record(cpu, what):
    """The cpu_baseline object of a JSON line from kv_oracle's timing."""
    many, one, cpus = cpu["many"], cpu["one"], cpu["cpus"]
    return {"value": round(many["GBps"], 3), "unit": "GB/s", "cores": many["threads"],
            "kind": "oracle", "cpu": cpu_model(),
            "single_thread_GBps": round(one["GBps"], 3), "nproc": cpus["nproc"],
            "affinity_cpus": cpus["affinity_cpus"], "cgroup_cpu_quota": cpus["cgroup_cpu_quota"],
            "sample": f"{what}: each thread a contiguous byte-balanced share of both directions' "
                      f"descriptors, per-descriptor memcpy between host images; median of "
                      f"{many['trials']} runs of {many['reps_per_trial']} steps on "
                      f"{many['threads']} threads ({many['seconds']:.1f} s), and of "
                      f"{one['trials']} runs of {one['reps_per_trial']} steps on 1 thread "
                      f"({one['seconds']:.1f} s)"}


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.strip().lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def check_kv_images(wl, final, imgs, what):
    """Exits with status 3 unless the device pool and the host D2H
    destination equal the oracle's images."""
    np = sys.modules["numpy"]
    for i in (0, 2):
        if not np.array_equal(final[i], imgs[i]):
            bad = int(np.flatnonzero(final[i] != imgs[i])[0])
            log(f"PARITY FAILURE{what} in arena {wl.arenas[i].name} at byte {bad}")
            sys.exit(3)


# ---------------------------------------------------------------------------
# Compact legs of the default run: mixed sizes (H2D) and the MoE gather
# ---------------------------------------------------------------------------

def mixed_compact(c: Ctx, args, ceil_h2d):
    """H2D with mixed 4-28 KiB sizes at N = 16, 256, 4,096, 65,536 (the
    vLLM PR #42212 report's small-block CPU->GPU case): per N the kernel-only
    rate (the kernel's own events), the rate of back-to-back calls, isolated
    per-call latency, and the kernel rate against the contiguous H2D
    ceiling measured in the same run; each N checked bit-exact against the
    oracle."""
    W, K = c.W, c.K
    g = ONE_WAY_MAX_WGS
    rows = {}
    for n in (16, 256, 4096, 65536):
        wl = W.h2d_mixed(seed=0, n=n)
        r = c.Resident(wl)
        b = wl.batches[0]
        pl = K.kvcopy_plan(*r.addrs[0], b.size)
        k = 100 if n <= 256 else 20 if n <= 4096 else 5
        s, _ = c.timed_bracketed(r, [0], [c.sA], k, min(args.leg_warmup, 10), g)
        _, km = c.timed(r, [0], [c.sA], k, 2, g)
        lat = c.latency(r, 0, g, k=30 if n <= 4096 else 5, w=3)
        c.verify(wl, r, [0], f"mixed {n}")
        kgb = gbs(b.nbytes, km[0] / 1e3)
        rows[str(n)] = {"bytes": b.nbytes, "merged": int(pl.n_merged), "chunks": int(pl.n_chunks),
                        "kernel_us": round(km[0] * 1e3, 2), "kernel_GBps": round(kgb, 2),
                        "back_to_back_GBps": round(gbs(b.nbytes, s), 2),
                        "frac_of_h2d_ceiling": round(kgb / ceil_h2d, 4) if ceil_h2d else None,
                        "latency": lat, "parity": "bit-exact vs oracle"}
        log(f"  mixed N={n}: {rows[str(n)]}")
        r.free()
    return {"max_wgs": g, "per_n": rows,
            "workload": "H2D, sizes 8-byte multiples in 4-28 KiB (70% in 8-16 KiB), 25% of "
                        "descriptors adjacent in both arenas, seed 0"}


def moe_upstream_order(b):
    """The descriptors of one MoE call bank-major (stable), for the
    upstream-style split: with one chunk per row, every wavefront gets the
    same number of rows and every bank the same number of wavefronts, so the
    1 MiB rows get a sixth of the workers (FreeToken issue #751, "Problem in
    upstream today")."""
    np = sys.modules["numpy"]
    return np.argsort(b.src_arena, kind="stable")


def moe_compact(c: Ctx, args, ceil_h2d, calls=20):
    """The MoE expert gather (26-39 experts x 6 bank rows per call, 3,164
    device slots): 20 calls per setting, byte-balanced 16 KiB chunks against
    the upstream-style split (equal workers per bank, bank-major, one chunk
    per row) at caps 1-8, plus byte-balanced at 32.  Every destination row
    written is checked against the oracle at the end, and untouched rows
    must keep the sentinel."""
    np, W, K = c.np, c.W, c.K
    wl = W.moe_gather(seed=0, calls=calls)
    r = c.Resident(wl)
    out = {}
    orders = [moe_upstream_order(b) for b in wl.batches]
    settings = [("byte_balanced_16KiB", g) for g in (1, 2, 4, 8, 32)] + \
               [("upstream_equal_workers_per_bank", g) for g in (1, 2, 4, 8)]
    for name, g in settings:
        t_us, sizes = [], []
        with no_gc():
            for i in range(calls):
                b = wl.batches[i]
                s_, d_ = r.addrs[i]
                if name.startswith("upstream"):
                    o = orders[i]
                    sub = lambda: K.kvcopy_batch(s_[o], d_[o], b.size[o], K.H2D, g,  # noqa: E731
                                                 c.sA.cuda_stream, chunk_bytes=K.CHUNK_MAX,
                                                 flags=K.F_NO_COALESCE)
                else:
                    sub = lambda: K.kvcopy_batch(s_, d_, b.size, K.H2D, g,  # noqa: E731
                                                 c.sA.cuda_stream)
                t_us.append(call_us(c, sub, c.sA))
                sizes.append(b.nbytes)
        rate = gbs(sum(sizes), sum(t_us) / 1e6)
        out[f"{name}/max_wgs={g}"] = {
            "call_us_p50": round(pct(t_us, 50), 1), "call_us_p99": round(pct(t_us, 99), 1),
            "GBps_total": round(rate, 2),
            "frac_of_h2d_ceiling": round(rate / ceil_h2d, 4) if ceil_h2d else None}
        log(f"  moe {name} max_wgs={g}: {out[f'{name}/max_wgs={g}']}")
    verify_moe_rows(c, wl, r, list(range(calls)))
    r.free()
    for g in (1, 2, 4, 8):
        bb = out[f"byte_balanced_16KiB/max_wgs={g}"]["GBps_total"]
        up = out[f"upstream_equal_workers_per_bank/max_wgs={g}"]["GBps_total"]
        out[f"speedup_byte_balanced_over_upstream/max_wgs={g}"] = round(bb / up, 3)
    out["parity"] = "every written row bit-exact vs oracle; sampled untouched rows keep the sentinel"
    return out


def verify_moe_rows(c: Ctx, wl, r, batch_ids, guard_rows=16):
    """Checks the MoE slot caches without reading 5.3 GB back: the oracle
    applies the calls to one image per written slot row (the rows start as
    the sentinel; later calls overwrite earlier ones as on the GPU), and the
    GPU's rows are gathered and compared with them; a few rows of each cache
    that no call wrote must still hold the sentinel.  Exits on mismatch."""
    import oracle
    np, torch = c.np, c.torch
    rows = wl.info["rows"]
    nb = len(rows)
    touched = {}                                   # cache arena -> sorted slots
    for k in batch_ids:
        b = wl.batches[k]
        for a, off in zip(b.dst_arena.tolist(), b.dst_off.tolist()):
            touched.setdefault(a, set()).add(off // rows[a - nb])
    touched = {a: sorted(v) for a, v in touched.items()}
    imgs = {(a, sl): np.full(rows[a - nb], wl.arenas[a].sentinel, np.uint8)
            for a, v in touched.items() for sl in v}
    srcs = [(r.bases[i], wl.arenas[i].host_image()) for i in range(nb)]
    dsts = [(r.bases[a] + sl * rows[a - nb], img) for (a, sl), img in imgs.items()]
    for k in batch_ids:
        b = wl.batches[k]
        s, d = r.addrs[k]
        oracle.copy(s, d, b.size, srcs, dsts)
    rng = np.random.default_rng(0)
    for a, slots in touched.items():
        row = rows[a - nb]
        view = r.bufs[a].view(-1, row)
        got = view[torch.tensor(slots, device=view.device)].cpu().numpy()
        for i, sl in enumerate(slots):
            if not np.array_equal(got[i], imgs[(a, sl)]):
                bad = int(np.flatnonzero(got[i] != imgs[(a, sl)])[0])
                log(f"PARITY FAILURE (moe rows) in {wl.arenas[a].name} slot {sl} at byte {bad}")
                sys.exit(3)
        free = np.setdiff1d(np.arange(view.shape[0]), slots)
        pick = rng.choice(free, size=min(guard_rows, len(free)), replace=False)
        g = view[torch.tensor(pick, device=view.device)].cpu().numpy()
        if not np.all(g == wl.arenas[a].sentinel):
            log(f"PARITY FAILURE (moe rows): an unwritten row of {wl.arenas[a].name} changed")
            sys.exit(3)


# ---------------------------------------------------------------------------
# The headline burst in one launch (kvcopy_batch_pair)
# ---------------------------------------------------------------------------

def bench_pair(c: Ctx, args):
    np, torch, W, K, hiprt = c.np, c.torch, c.W, c.K, c.hiprt
    wl = W.kv_blocks(seed=0, directions="both")
    res = c.Resident(wl)
    step_bytes = wl.nbytes
    g = args.max_wgs if args.max_wgs is not None else K.WGS_AUTO
    log(f"pair: {sum(b.n for b in wl.batches)} descriptors in one call, max_wgs={g}")
    # settle the host link first, as the headline does, then the --warmup steps
    t_settle, done = time.perf_counter(), 0
    while done < LINK_SETTLE_STEPS and time.perf_counter() - t_settle < LINK_SETTLE_SECONDS:
        for _ in range(50):
            c.pair_step(res, c.sA, g)
        hiprt.stream_sync(c.sA)
        done += 50
    for _ in range(args.warmup):
        c.pair_step(res, c.sA, g)
    torch.cuda.synchronize()
    use_ev = not args.no_events
    e0, e1 = (hiprt.Event(), hiprt.Event()) if use_ev else (None, None)
    with no_gc():
        t0 = time.perf_counter()
        if use_ev:
            e0.record(c.sA)
        for _ in range(args.steps):
            c.pair_step(res, c.sA, g)
        if use_ev:
            e1.record(c.sA)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    # The launches run back to back on one stream: the event pair around
    # them, divided by the steps, is the mean kernel duration.
    kern_ms = e0.elapsed_ms(e1) / args.steps if use_ev else step_s * 1e3
    value = gbs(step_bytes, step_s)
    log(f"  one launch: {step_s * 1e3:.3f} ms/step, {value:.2f} GB/s; kernel {kern_ms:.4f} ms")
    chunks = sum(K.kvcopy_plan(*res.addrs[j], wl.batches[j].size).n_chunks for j in range(2))
    alg_fetch = step_bytes + chunks * REC_BYTES       # both payloads read + the worklist records
    alg_write = step_bytes
    ach = gbs(alg_fetch, kern_ms / 1e3)   # bytes over the host link: payload both ways + records
    extras = {}
    if not args.skip_extras:
        # the two-stream submission of the same burst first: it also brings
        # both streams into use before the contiguous ceilings are taken on them
        hA, hB, _ = c.headline_streams()
        extras["two_streams_same_run_GBps"] = round(gbs(step_bytes, c.timed_bracketed(
            res, [0, 1], [hA, hB], args.steps, args.leg_warmup, DEFAULT_MAX_WGS,
            joined=True)[0]), 3)
        extras["contiguous_memcpy_ceiling_GBps"] = ceilings(c)
        log(f"  ceilings {extras['contiguous_memcpy_ceiling_GBps']}, two streams at "
            f"{DEFAULT_MAX_WGS}: {extras['two_streams_same_run_GBps']} GB/s")
    if args.counter_calibration:
        counter_calibration(c)
    res.fill()
    c.pair_step(res, c.sA, g)
    torch.cuda.synchronize()
    final = {i: res.image(i) for i in (0, 2)}
    imgs, cpu = kv_oracle(c, wl, res, args)
    check_kv_images(wl, final, imgs, " (one launch)")
    log("  parity: bit-exact against the oracle")
    res.free()
    meas_ceil = extras.get("contiguous_memcpy_ceiling_GBps", {}).get("both")
    line = base_line(args, round(value, 3), "GB/s", step_s, {
        "workload": "bidirectional KV block burst in one launch: 16,384 shuffled 4 KiB H2D + "
                    "16,384 shuffled 4 KiB D2H per step as one kvcopy_batch_pair call on one "
                    "stream, 65,536-block device pool, mapped pinned host buffers",
        "descriptors_per_step": sum(b.n for b in wl.batches), "bytes_per_step": step_bytes,
        "max_wgs": g, "chunk_bytes": K.CHUNK_DEFAULT, "seed": 0})
    line["roofline"] = {
        "bound": "pcie", "kernel": "kvcopy_pair_kernel", "achieved": round(ach, 3),
        "peak": 2 * PCIE_PEAK_GBS, "unit": "GB/s", "frac": round(ach / (2 * PCIE_PEAK_GBS), 4),
        "traffic": measured_traffic("kvcopy_pair_kernel", COUNTERS_PAIR, alg_fetch, alg_write),
        "kernel_ms": round(kern_ms, 4), "algorithmic_bytes_per_launch": alg_fetch,
        "peak_note": "both directions of PCIe 5.0 x16 (64 GB/s each)", "link": pcie_link(),
        "measured_ceiling": meas_ceil,
        "frac_of_measured_ceiling": round(ach / meas_ceil, 4) if meas_ceil else None}
    line["cpu_baseline"] = cpu_baseline_record(
        cpu, "whole steps of 16,384 H2D + 16,384 D2H descriptors of 4 KiB")
    line["parity"] = "bit-exact vs oracle"
    line.update(extras)
    return line


def pair_rates(c: Ctx, res, args):
    """The headline step as one kvcopy_batch_pair call per step (both lists
    in one launch on one stream), at a few workgroup caps: GB/s of payload
    over k back-to-back calls bracketed by one event pair."""
    torch, hiprt = c.torch, c.hiprt
    step_bytes = res.wl.nbytes
    out = {}
    for g in (32, 48, 64, 80, 128, 256, 0):
        for _ in range(args.leg_warmup):
            c.pair_step(res, c.sA, g)
        torch.cuda.synchronize()
        use_ev = not args.no_events
        e0, e1 = (hiprt.Event(), hiprt.Event()) if use_ev else (None, None)
        with no_gc():
            t0 = time.perf_counter()
            if use_ev:
                e0.record(c.sA)
            for _ in range(args.steps):
                c.pair_step(res, c.sA, g)
            if use_ev:
                e1.record(c.sA)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        ms = e0.elapsed_ms(e1) / args.steps if use_ev else (t1 - t0) / args.steps * 1e3
        out[str(g)] = {"GBps": round(gbs(step_bytes, ms / 1e3), 3), "ms_per_step": round(ms, 4),
                       "wall_GBps": round(gbs(step_bytes, (t1 - t0) / args.steps), 3)}
        log(f"  one-launch pair max_wgs={g}: {out[str(g)]}")
    return out


def counter_calibration(c: Ctx):
    """A plain elementwise kernel of known traffic (reads 64 MiB, writes 64 MiB),
    run 5 times, whose PMC byte counts scale those of the copy kernels."""
    torch = c.torch
    a = torch.arange(16 * c.W.MIB, dtype=torch.int32, device=c.dev)
    b = torch.empty_like(a)
    for _ in range(5):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def ceilings(c: Ctx, nb=None, reps=10):
    """Contiguous hipMemcpyAsync of 64 MiB from/to mapped pinned memory, per
    direction and both together on two streams (GB/s, median of reps)."""
    torch, hiprt, K, W = c.torch, c.hiprt, c.K, c.W
    nb = nb or 64 * W.MIB
    hsrc, hdst = K.HostBuffer(nb), K.HostBuffer(nb)
    hsrc.array[:] = 7
    dbuf = torch.empty(2 * nb, dtype=torch.uint8, device=c.dev)

    def one(kinds):
        times = []
        for r in range(reps + 2):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i, kind in enumerate(kinds):
                st = (c.sA, c.sB)[i]
                if kind == "h2d":
                    hiprt.memcpy_async(dbuf.data_ptr(), hsrc.ptr, nb, hiprt.H2D_KIND, st)
                else:
                    hiprt.memcpy_async(hdst.ptr, dbuf.data_ptr() + nb, nb, hiprt.D2H_KIND, st)
            torch.cuda.synchronize()
            if r >= 2:
                times.append(time.perf_counter() - t0)
        return round(gbs(nb * len(kinds), statistics.median(times)), 3)

    out = {"h2d": one(["h2d"]), "d2h": one(["d2h"]), "both": one(["h2d", "d2h"])}
    del dbuf
    hsrc.free()
    hdst.free()
    return out


def per_fragment(c: Ctx, plan, kind, reps=2):
    """Seconds per batch for one hipMemcpyAsync per (coalesced) range on one stream."""
    torch, hiprt = c.torch, c.hiprt
    srcs, dsts, sizes = plan.src.tolist(), plan.dst.tolist(), plan.size.tolist()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        for s_, d_, z_ in zip(srcs, dsts, sizes):
            hiprt.memcpy_async(d_, s_, z_, kind, c.sA)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps


# The C-caller tool's header flag that makes it time one hipMemcpyAsync per
# range instead of kvcopy_batch (latency_tool.cpp, kRuntimeCopy).
RUNTIME_COPY_FLAG = 0x80000000


def c_caller_latency(named):
    """Per-call latency of kvcopy_batch from a C caller: block_copy_amd/kvcopy_latency
    (built with the library) in a child process without torch, so the figures
    carry no Python marshalling.  `named` is a list of (name, workload,
    max_wgs) with one batch each, between one source and one destination
    arena; the child allocates its own arenas of the same sizes, times
    isolated and back-to-back calls, and checks every destination range
    against its source.  Returns {name: row}, with an "error" entry if the
    tool is missing or fails."""
    import struct
    import subprocess
    import tempfile
    exe = os.path.join(ROOT, "block_copy_amd", "kvcopy_latency")
    if not os.path.exists(exe):
        return {"error": "block_copy_amd/kvcopy_latency is not built"}
    with tempfile.TemporaryDirectory() as td:
        files = []
        for entry in named:
            name, wl, max_wgs = entry[:3]
            flags = entry[3] if len(entry) > 3 else 0
            b = wl.batches[0]
            if len(set(b.src_arena.tolist())) != 1 or len(set(b.dst_arena.tolist())) != 1:
                raise ValueError(f"{name}: one source and one destination arena expected")
            sa, da = wl.arenas[int(b.src_arena[0])], wl.arenas[int(b.dst_arena[0])]
            path = os.path.join(td, f"{name}.bin")
            with open(path, "wb") as f:
                f.write(struct.pack("<64sIIiIQQQ", name.encode()[:63], sa.where == "host",
                                    da.where == "host", int(max_wgs), int(flags), sa.nbytes,
                                    da.nbytes, b.n))
                for a in (b.src_off, b.dst_off, b.size):
                    f.write(a.astype("<u8").tobytes())
            files.append(path)
        try:
            r = subprocess.run([exe, *files], capture_output=True, text=True, timeout=600)
        except subprocess.TimeoutExpired:
            return {"error": "kvcopy_latency timed out"}
    rows = {}
    for line in r.stdout.splitlines():
        row = json.loads(line)
        rows[row.pop("name")] = row
    if r.returncode != 0:
        rows["error"] = f"kvcopy_latency exited with {r.returncode}: {r.stderr.strip()[-300:]}"
    return rows


def dma_runtime_baselines():
    """The DMA baselines of block_copy_amd/dma_baselines.py, run in a child
    process without torch (on ROCm's own HIP runtime, which exports
    hipMemcpyBatchAsync); None if the child fails."""
    import subprocess
    try:
        r = subprocess.run([sys.executable, "-m", "block_copy_amd.dma_baselines"], cwd=ROOT,
                           capture_output=True, text=True, timeout=300)
    except subprocess.TimeoutExpired:
        log("  DMA baselines child timed out")
        return None
    for ln in r.stderr.splitlines():
        if "amdgpu.ids" not in ln:
            log(f"  [dma child] {ln}")
    if r.returncode != 0:
        log(f"  DMA baselines child exited with {r.returncode}")
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def dma_baselines(c: Ctx, plan, nbytes, kind, reps=2):
    """One hipMemcpyAsync per (coalesced) range on one stream, in this process
    (on the HIP runtime the kernel runs on)."""
    dt = per_fragment(c, plan, kind, reps=reps)
    return {"per_fragment": {"GBps": round(gbs(nbytes, dt), 3), "ms_per_call": round(dt * 1e3, 3),
                             "copies": int(plan.n_merged)}}


# ---------------------------------------------------------------------------
# D2D
# ---------------------------------------------------------------------------

def d2d_results(c: Ctx, args):
    torch, W, K, hiprt = c.torch, c.W, c.K, c.hiprt
    out = {}
    for name, wld in (("1024x4KiB", W.d2d_blocks(seed=0)),
                      ("65536x4KiB", W.d2d_blocks(seed=1, n=65536, pool_blocks=262144))):
        r = c.Resident(wld)
        # back-to-back calls with no per-launch event (call rate), then the
        # same calls with the kernel's own start/end events (kernel time)
        s, stream_ms = c.timed_bracketed(r, [0], [c.sA], args.steps, args.leg_warmup, 0)
        _, km = c.timed(r, [0], [c.sA], args.steps, 2, 0)
        pl = K.kvcopy_plan(*r.addrs[0], wld.batches[0].size)
        hbm = 2 * wld.batches[0].nbytes + pl.n_chunks * REC_BYTES
        out[name] = {"payload_bytes": wld.batches[0].nbytes, "records": int(pl.n_chunks),
                     "GBps_payload": round(gbs(wld.batches[0].nbytes, s), 2),
                     "us_per_call_pipelined": round(s * 1e6, 2),
                     "gpu_us_per_call_back_to_back": round(stream_ms[0] * 1e3, 2),
                     "kernel_us": round(km[0] * 1e3, 2),
                     "hbm_GBps_kernel": round(gbs(hbm, km[0] / 1e3), 1),
                     "frac_hbm_peak_kernel": round(gbs(hbm, km[0] / 1e3) / HBM_PEAK_GBS, 4),
                     "latency": c.latency(r, 0, 0, k=200 if name == "1024x4KiB" else 50,
                                          w=20 if name == "1024x4KiB" else 5)}
        out[name]["mall_flushed"] = d2d_flushed(c, r, k=max(20, args.steps))
        c.verify(wld, r, [0], f"d2d {name}")
        if name == "65536x4KiB" and not args.no_events:
            # the workgroup-per-chunk mode on the same call, parity-checked
            # (profiler runs see that kernel on distinct calls only, below)
            r.fill()
            for _ in range(5):
                r.submit(0, 0, c.sA, flags=K.F_WG_PER_CHUNK | K.F_DESC_UPLOAD | K.F_DST_ORDER)
            hiprt.stream_sync(c.sA)
            c.verify(wld, r, [0], f"d2d {name}, workgroup per chunk")
        if name == "65536x4KiB":
            out[name]["note"] = ("kernel_us: the same call repeated, so most of its 256 MiB of "
                                 "sources stay in the 256 MB MALL between calls")
        if name == "1024x4KiB":     # after the check: the DMA baselines write the same bytes
            if not args.no_events:
                out[name]["launch_floor_and_caps"] = d2d_launch_floor(c, r)
                log(f"  d2d {name} kernel vs empty-kernel floor: "
                    f"{out[name]['launch_floor_and_caps']}")
            out[name]["dma_baselines"] = dma_baselines(c, pl, wld.batches[0].nbytes,
                                                       hiprt.D2D_KIND, reps=5)
            out[name]["latency_c_caller"] = c_caller_latency([("d2d_1024x4KiB", wld, 0)]).get(
                "d2d_1024x4KiB")
        else:
            cl = c_caller_latency([("d2d_65536x4KiB", wld, 0),
                                   ("d2d_65536x4KiB_dst_order", wld, 0, K.F_DST_ORDER),
                                   ("d2d_65536x4KiB_wg_dst_order_upload", wld, 0,
                                    K.F_DST_ORDER | K.F_DESC_UPLOAD | K.F_WG_PER_CHUNK)])
            out[name]["latency_c_caller"] = cl.get("d2d_65536x4KiB", cl.get("error"))
            out[name]["latency_c_caller_dst_order"] = cl.get("d2d_65536x4KiB_dst_order",
                                                             cl.get("error"))
            out[name]["latency_c_caller_wg_dst_order_upload"] = cl.get(
                "d2d_65536x4KiB_wg_dst_order_upload", cl.get("error"))
        log(f"  d2d {name}: {out[name]} (bit-exact)")
        r.free()
    big = torch.empty(2 << 30, dtype=torch.uint8, device=c.dev)
    cont = {}
    for nbytes in (256 << 20, 1 << 30):
        ms = []
        for _ in range(5):
            if args.no_events:          # profiler runs: wall clock around a synchronised copy
                hiprt.stream_sync(c.sA)
                t0 = time.perf_counter()
                hiprt.memcpy_async(big.data_ptr() + (1 << 30), big.data_ptr(), nbytes, hiprt.D2D_KIND, c.sA)
                hiprt.stream_sync(c.sA)
                ms.append((time.perf_counter() - t0) * 1e3)
                continue
            e1, e2 = hiprt.Event(), hiprt.Event()
            e1.record(c.sA)
            hiprt.memcpy_async(big.data_ptr() + (1 << 30), big.data_ptr(), nbytes, hiprt.D2D_KIND, c.sA)
            e2.record(c.sA)
            ms.append(e1.elapsed_ms(e2))
        cont[f"{nbytes >> 20}MiB"] = round(gbs(2 * nbytes, statistics.median(ms) / 1e3), 1)
    out["contiguous_memcpy_hbm_GBps"] = cont
    log(f"  contiguous D2D hipMemcpyAsync (HBM GB/s): {cont}")
    if not args.no_events:
        # the same kernel on one contiguous range (chunked into 16 KiB pieces):
        # what scatter/gather costs against a plain copy of the same bytes
        # (1 GiB also with 2 KiB chunks and the worklist uploaded first, the
        # fastest contiguous copy measured with this kernel: more, shorter
        # wavefronts, and 512 Ki records read from HBM instead of the host link)
        kc = {}
        for key, nbytes, chunk, flags in (("256MiB", 256 << 20, 0, 0), ("1024MiB", 1 << 30, 0, 0),
                                          ("1024MiB_chunk2KiB_uploaded", 1 << 30, 2048,
                                           K.F_DESC_UPLOAD)):
            s_ = c.np.array([big.data_ptr()], c.np.uint64)
            d_ = c.np.array([big.data_ptr() + (1 << 30)], c.np.uint64)
            z_ = c.np.array([nbytes], c.np.uint64)
            ev = (hiprt.Event(), hiprt.Event())
            ms = []
            for i in range(8):
                K.kvcopy_batch(s_, d_, z_, K.D2D, 0, c.sA.cuda_stream, chunk_bytes=chunk,
                               flags=flags, kernel_begin=ev[0].h, kernel_end=ev[1].h)
                if i >= 2:
                    ms.append(ev[0].elapsed_ms(ev[1]))
            kc[key] = round(gbs(2 * nbytes, statistics.median(ms) / 1e3), 1)
        out["kernel_one_contiguous_range_hbm_GBps"] = kc
        log(f"  the kernel on one contiguous range (HBM GB/s): {kc}")
    del big
    out["65536x4KiB"]["distinct_calls"] = d2d_distinct(c, args)
    return out


def headline_windows(c: Ctx, res, max_wgs, n=30, k=20, streams=None, **kw):
    """n consecutive windows of k joined steps of the headline burst (the
    step count the headline is timed over) on `streams` (default sA, sB),
    each timed by wall clock around the window and by one event pair per
    stream around its kernels: the spread of the two-stream rate, and in
    each window whether both kernels slowed or one stream ran longer than
    the other."""
    step_bytes = res.wl.nbytes
    st = list(streams) if streams is not None else [c.sA, c.sB]
    rates, kern = [], []
    for _ in range(n):
        s, km = c.timed_bracketed(res, [0, 1], st, k, 0, max_wgs, joined=True, **kw)
        rates.append(gbs(step_bytes, s))
        kern.append([round(x, 4) for x in km])
    med = statistics.median(rates)
    within = sum(1 for x in rates if abs(x / med - 1) <= 0.03)
    return {"windows": n, "steps_per_window": k, "GBps_median": round(med, 3),
            "GBps_min": round(min(rates), 3), "GBps_max": round(max(rates), 3),
            "within_3pct_of_median": within, "GBps": [round(x, 2) for x in rates],
            "kernel_ms_per_stream": kern}


def d2d_launch_floor(c: Ctx, r, grids=(16, 32, 64, 128, 256), reps=50):
    """The 1,024 x 4 KiB call's kernel time at caps 16-256 (the default loop
    choice: pipelined at 16-128, where every wavefront has 2-16 chunks; at
    256, the full grid, one chunk per wavefront) beside an empty kernel of
    the same grid, both from the kernels' own events in this run (median of
    `reps` launches each)."""
    from block_copy_amd import decode_load as DL
    hiprt = c.hiprt
    out = {}
    for g in grids:
        evs = [(hiprt.Event(), hiprt.Event()) for _ in range(reps)]
        for e0, e1 in evs:
            DL.empty(g, c.sA, e0.h, e1.h)
        floor = statistics.median(e0.elapsed_ms(e1) * 1e3 for e0, e1 in evs)
        evs = [(hiprt.Event(), hiprt.Event()) for _ in range(reps)]
        for e0, e1 in evs:
            r.submit(0, g, c.sA, kernel_begin=e0.h, kernel_end=e1.h)
        us = statistics.median(e0.elapsed_ms(e1) * 1e3 for e0, e1 in evs)
        out[f"max_wgs={g}"] = {"kernel_us_p50": round(us, 2),
                               "empty_kernel_us_p50_same_grid": round(floor, 2),
                               "kernel_minus_floor_us": round(us - floor, 2)}
    best = min(out, key=lambda k: out[k]["kernel_us_p50"])
    out["best"] = best
    return out


def d2d_flushed(c: Ctx, r, k=20):
    """The gather with the 256 MB MALL (Infinity Cache) holding none of its
    bytes: a kernel that reads 512 MiB of other memory runs on the same stream
    before every call, outside the kernel's own start/end events.  The scrub
    only reads, so it leaves no dirty lines whose write-back would land inside
    the timed kernel.  Returns the median kernel time and the HBM rate it
    implies, and the per-call GPU time."""
    torch, hiprt = c.torch, c.hiprt
    if c.args.no_events:
        return None
    scrub = torch.zeros(512 << 20, dtype=torch.uint8, device=c.dev).view(torch.int32)
    kern, call = [], []
    with torch.cuda.stream(c.sA):
        for i in range(k + 3):
            scrub.max()
            e0, e1, k0, k1 = hiprt.Event(), hiprt.Event(), hiprt.Event(), hiprt.Event()
            e0.record(c.sA)
            r.submit(0, 0, c.sA, kernel_begin=k0.h, kernel_end=k1.h)
            e1.record(c.sA)
            if i >= 3:
                kern.append(k0.elapsed_ms(k1) * 1e3)
                call.append(e0.elapsed_ms(e1) * 1e3)
    c.sA.synchronize()
    del scrub
    nbytes = r.wl.batches[0].nbytes
    kt = statistics.median(kern)
    return {"kernel_us_p50": round(kt, 2), "hbm_GBps_kernel": round(gbs(2 * nbytes, kt / 1e6), 1),
            "gpu_us_p50": round(statistics.median(call), 2), "calls": k,
            "scrub": "512 MiB read on the same stream before each call"}


def d2d_distinct(c: Ctx, args):
    """65,536 x 4 KiB D2D calls that cycle through 8 different batches over the
    same two 1 GiB pools (W.d2d_rotation), so that each call's bytes are
    mostly not in the MALL and the write-backs of earlier calls land in later
    ones, as in a long run of distinct calls.  Kernel-only time from each
    kernel's own events; the final images are checked against the oracle
    applying the 8 batches in order."""
    torch, hiprt, W = c.torch, c.hiprt, c.W
    wl = W.d2d_rotation()
    r = c.Resident(wl)
    nb = len(wl.batches)
    if args.no_events:
        # profiler runs: the library's own fast mode for an unsorted list
        # (one workgroup per chunk, records uploaded and grouped by
        # destination region on the GPU, sc1 stores), timed by the kernel
        # trace (its kernels, kvcopy_order_count_kernel,
        # kvcopy_order_place_kernel and kvcopy_d2d_wg_sc1_kernel, run nowhere
        # else in a profiled D2D leg), parity-checked
        K = c.K
        fl = K.F_WG_PER_CHUNK | K.F_DESC_UPLOAD | K.F_DST_ORDER | K.F_STORE_SC1
        calls = max(4 * nb, args.steps)
        r.fill()
        for i in range(nb):
            r.submit(i, 0, c.sA, flags=fl)
        hiprt.stream_sync(c.sA)
        c.verify(wl, r, list(range(nb)), "d2d distinct calls, workgroup per chunk")
        for i in range(calls):
            r.submit(i % nb, 0, c.sA, flags=fl)
        hiprt.stream_sync(c.sA)
        r.free()
        return {"calls": calls, "mode": "KVCOPY_F_WG_PER_CHUNK | KVCOPY_F_DESC_UPLOAD | "
                "KVCOPY_F_DST_ORDER | KVCOPY_F_STORE_SC1",
                "timed_by": "the kernel trace (kvcopy_d2d_wg_sc1_kernel)"}
    calls = max(4 * nb, args.steps)

    K = c.K
    # each batch's descriptors sorted by destination address on the caller's
    # side (the copy's result does not depend on the order: no destination
    # overlaps another within a batch)
    by_dst = []
    for i in range(nb):
        s_, d_ = r.addrs[i]
        o = c.np.argsort(d_, kind="stable")
        by_dst.append((s_[o], d_[o], wl.batches[i].size[o]))

    def kernel_us(flags, sorted_=False):
        evs = [(hiprt.Event(), hiprt.Event()) for _ in range(calls)]

        def call(i, **kw):
            if sorted_:
                s_, d_, z_ = by_dst[i]
                K.kvcopy_batch(s_, d_, z_, W.D2D, 0, c.sA.cuda_stream, flags=flags, **kw)
            else:
                r.submit(i, 0, c.sA, flags=flags, **kw)

        for i in range(nb):
            call(i)
        for i in range(calls):
            call(i % nb, kernel_begin=evs[i][0].h, kernel_end=evs[i][1].h)
        hiprt.stream_sync(c.sA)
        return [e0.elapsed_ms(e1) * 1e3 for e0, e1 in evs]

    # list order and destination order, alternating twice so that drift over
    # the run falls on both alike
    t_list, t_dst = [], []
    for _ in range(2):
        t_list += kernel_us(0)
        t_dst += kernel_us(K.F_DST_ORDER)
    us, us_dst = statistics.median(t_list), statistics.median(t_dst)
    # where the records live and how the caller orders the list: records
    # uploaded to device memory before each kernel (KVCOPY_F_DESC_UPLOAD),
    # the list sorted by destination, and both, with either store form
    # and the workgroup-per-chunk loop (KVCOPY_F_WG_PER_CHUNK), which reads
    # each chunk's record in its workgroup and so wants them in device memory
    WG = K.F_WG_PER_CHUNK | K.F_DESC_UPLOAD
    variants = {"list_order_records_in_device_memory": (K.F_DESC_UPLOAD, False),
                "sorted_by_destination": (0, True),
                "sorted_by_destination_records_in_device_memory": (K.F_DESC_UPLOAD, True),
                "sorted_by_destination_records_in_device_memory_sc1_stores":
                    (K.F_DESC_UPLOAD | K.F_STORE_SC1, True),
                "wg_per_chunk_records_in_device_memory": (WG, False),
                "wg_per_chunk_destination_order_records_in_device_memory": (WG | K.F_DST_ORDER, False),
                "wg_per_chunk_destination_order_records_in_device_memory_sc1_stores":
                    (WG | K.F_DST_ORDER | K.F_STORE_SC1, False),
                "wg_per_chunk_sorted_by_destination_records_in_device_memory": (WG, True),
                "wg_per_chunk_sorted_by_destination_records_in_device_memory_sc1_stores":
                    (WG | K.F_STORE_SC1, True)}
    var_us = {name: [] for name in variants}
    for _ in range(2):
        for name, (fl, srt) in variants.items():
            var_us[name] += kernel_us(fl, srt)
    pl = c.K.kvcopy_plan(*r.addrs[0], wl.batches[0].size)
    hbm = 2 * wl.batches[0].nbytes + pl.n_chunks * REC_BYTES
    ceiling = random_block_ceiling(c, r, wl, calls)
    r.fill()
    for i in range(nb):
        r.submit(i, 0, c.sA, flags=c.K.F_DST_ORDER)
    hiprt.stream_sync(c.sA)
    c.verify(wl, r, list(range(nb)), "d2d distinct calls, destination order")
    r.fill()
    for i in range(nb):
        s_, d_, z_ = by_dst[i]
        K.kvcopy_batch(s_, d_, z_, W.D2D, 0, c.sA.cuda_stream,
                       flags=K.F_DESC_UPLOAD | K.F_STORE_SC1)
    hiprt.stream_sync(c.sA)
    c.verify(wl, r, list(range(nb)), "d2d distinct calls, sorted, uploaded records, sc1 stores")
    r.fill()
    for i in range(nb):
        r.submit(i, 0, c.sA, flags=WG | K.F_DST_ORDER)
    hiprt.stream_sync(c.sA)
    c.verify(wl, r, list(range(nb)), "d2d distinct calls, workgroup per chunk, destination order")
    # back-to-back calls in the workgroup mode, the record upload included:
    # GPU time per call between two events around all calls
    e0, e1 = hiprt.Event(), hiprt.Event()
    per_call = {}
    def call_sorted(i, fl):
        s_, d_, z_ = by_dst[i]
        K.kvcopy_batch(s_, d_, z_, W.D2D, 0, c.sA.cuda_stream, flags=fl)

    for name, fl, srt in (("list_order_default", 0, False),
                          ("wg_per_chunk_destination_order_records_uploaded",
                           WG | K.F_DST_ORDER, False),
                          ("wg_per_chunk_destination_order_records_uploaded_sc1_stores",
                           WG | K.F_DST_ORDER | K.F_STORE_SC1, False),
                          ("wg_per_chunk_sorted_by_destination_records_uploaded", WG, True),
                          ("wg_per_chunk_sorted_by_destination_records_uploaded_sc1_stores",
                           WG | K.F_STORE_SC1, True)):
        def call(i):
            if srt:
                call_sorted(i, fl)
            else:
                r.submit(i, 0, c.sA, flags=fl)
        for i in range(nb):
            call(i)
        e0.record(c.sA)
        for i in range(calls):
            call(i % nb)
        e1.record(c.sA)
        per_call[name] = round(e0.elapsed_ms(e1) * 1e3 / calls, 2)
    r.fill()
    for i in range(nb):
        r.submit(i, 0, c.sA)
    hiprt.stream_sync(c.sA)
    c.verify(wl, r, list(range(nb)), "d2d distinct calls")
    r.free()
    out = {"batches": nb, "calls": calls, "kernel_us_p50": round(us, 2),
           "hbm_GBps_kernel": round(gbs(hbm, us / 1e6), 1),
           "frac_hbm_peak_kernel": round(gbs(hbm, us / 1e6) / HBM_PEAK_GBS, 4),
           "destination_order": {"kernel_us_p50": round(us_dst, 2),
                                 "hbm_GBps_kernel": round(gbs(hbm, us_dst / 1e6), 1),
                                 "frac_hbm_peak_kernel": round(gbs(hbm, us_dst / 1e6) / HBM_PEAK_GBS, 4),
                                 "flag": "KVCOPY_F_DST_ORDER", "parity": "bit-exact vs oracle"},
           "random_block_ceiling": ceiling,
           "frac_random_block_ceiling": round(ceiling["us"] / us, 4)}
    out["gpu_us_per_call_back_to_back"] = per_call
    for name, v in var_us.items():
        u = statistics.median(v)
        out[name] = {"kernel_us_p50": round(u, 2), "hbm_GBps_kernel": round(gbs(hbm, u / 1e6), 1),
                     "frac_hbm_peak_kernel": round(gbs(hbm, u / 1e6) / HBM_PEAK_GBS, 4)}
        fl = variants[name][0]
        if fl & K.F_DST_ORDER and fl & K.F_DESC_UPLOAD:
            # the kernel events bracket the copy kernel; the grouping runs
            # before it, on the library's upload stream (its kernels are in
            # the D2D kernel trace), and is inside the back-to-back figures
            out[name]["events_cover"] = ("the copy kernel; the order kernels run before it on the "
                                         "library's upload stream")
    log(f"  d2d distinct calls: {out} (bit-exact)")
    return out


def random_block_ceiling(c: Ctx, r, wl, calls):
    """What HBM sustains for the rotation's own blocks moved one way at a time:
    the same source blocks only read, and the same destination blocks only
    written (libkvload's scattered passes: one wavefront per block, the copy's
    access shapes), each timed per launch with the kernel's own events, the
    calls cycling over the batches as the copy's do.  Reads and writes share
    each HBM channel's data bus, so the copy cannot beat read time + write
    time; that sum, against 2 x payload, is the random-block ceiling.  Runs
    after the copy calls and before the refill that precedes the check (the
    scatter overwrites destination blocks)."""
    torch, hiprt, np = c.torch, c.hiprt, c.np
    from block_copy_amd import decode_load as DL
    sizes = {int(x) for b in wl.batches for x in np.unique(b.size)}
    if len(sizes) != 1:
        raise ValueError("the random-block ceiling needs one block size")
    blk = sizes.pop()
    nb = len(wl.batches)
    srcs = [torch.from_numpy(r.addrs[i][0].view(np.int64)).to(c.dev) for i in range(nb)]
    dsts = [torch.from_numpy(r.addrs[i][1].view(np.int64)).to(c.dev) for i in range(nb)]
    sink = torch.zeros(64, dtype=torch.int32, device=c.dev)
    res = {}
    for kind in ("read", "write"):
        def launch(i, e0=None, e1=None):
            if kind == "read":
                DL.gather_read(srcs[i % nb], blk, sink, c.sA, e0, e1)
            else:
                DL.scatter_write(dsts[i % nb], blk, 0xA5A5A5A5, c.sA, e0, e1)
        for i in range(nb):
            launch(i)
        evs = [(hiprt.Event(), hiprt.Event()) for _ in range(calls)]
        for i in range(calls):
            launch(i, evs[i][0].h, evs[i][1].h)
        hiprt.stream_sync(c.sA)
        res[kind] = statistics.median(e0.elapsed_ms(e1) * 1e3 for e0, e1 in evs)
    payload = wl.batches[0].nbytes
    us = res["read"] + res["write"]
    return {"us": round(us, 2), "GBps": round(gbs(2 * payload, us / 1e6), 1),
            "read_only_us_p50": round(res["read"], 2),
            "read_only_GBps": round(gbs(payload, res["read"] / 1e6), 1),
            "write_only_us_p50": round(res["write"], 2),
            "write_only_GBps": round(gbs(payload, res["write"] / 1e6), 1),
            "what": "the same random 4 KiB blocks only read, then only written, each pass "
                    "timed alone; ceiling = 2 x payload / (read time + write time)"}


def bench_d2d(c: Ctx, args):
    res = d2d_results(c, args)
    if args.counter_calibration:
        counter_calibration(c)
    r1 = res["1024x4KiB"]
    # A 4 MiB call takes a few microseconds on the GPU, so back-to-back calls
    # from Python are bound by the interpreter (about 10 us of marshalling
    # per call).  The value is therefore the same calls made back to back
    # from C (kvcopy_latency, in a child process); the Python rate is kept.
    cc = r1.get("latency_c_caller") or {}
    if cc.get("pipelined_us_per_call") and not cc.get("ranges_wrong"):
        us = cc["pipelined_us_per_call"]
        value, src = round(gbs(r1["payload_bytes"], us / 1e6), 2), "C caller, back-to-back calls"
    else:
        us, value, src = r1["us_per_call_pipelined"], r1["GBps_payload"], "Python, back-to-back calls"
    line = base_line(args, value, "GB/s", us / 1e6, {
        "workload": "D2D gather/scatter of 1,024 x 4 KiB blocks between two 4,096-block pools; "
                    "also 65,536 x 4 KiB between two 1 GiB pools",
        "max_wgs": 0, "chunk_bytes": c.K.CHUNK_DEFAULT, "seed": 0})
    line["value_source"] = src
    if src.startswith("C"):
        line["value_calls"] = cc.get("pipelined_calls", cc["calls"])
    line["value_python_GBps"] = r1["GBps_payload"]
    big = res["65536x4KiB"]
    dist = big.get("distinct_calls")
    if dist is not None and "hbm_GBps_kernel" not in dist:
        dist = None        # profiler runs: those calls are timed by the trace
    # The roofline is taken on calls over distinct blocks: repeating one call
    # lets the MALL serve most of its sources.  The practical ceiling is a
    # contiguous copy with a 2 GiB footprint (beyond the MALL), by DMA or by
    # this kernel on one range.
    kc = res.get("kernel_one_contiguous_range_hbm_GBps", {})
    ceil = max(res["contiguous_memcpy_hbm_GBps"]["1024MiB"], kc.get("1024MiB", 0.0),
               kc.get("1024MiB_chunk2KiB_uploaded", 0.0))
    ach = dist["hbm_GBps_kernel"] if dist else big["hbm_GBps_kernel"]
    line["roofline"] = {"bound": "hbm", "kernel": kernel_name(2, args.store),
                        "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(kernel_name(2, args.store), COUNTERS_D2D,
                                                    big["payload_bytes"] + big["records"] * REC_BYTES,
                                                    big["payload_bytes"]),
                        "workload_of_roofline": "65536x4KiB, calls cycling over 8 distinct batches"
                                                if dist else "65536x4KiB, one call repeated",
                        "achieved_one_call_repeated": big["hbm_GBps_kernel"],
                        "measured_ceiling": ceil,
                        "measured_ceiling_what": "contiguous 1 GiB D2D copy (2 GiB footprint): the "
                                                 "best of hipMemcpyAsync and this kernel on one range",
                        "frac_of_measured_ceiling": round(ach / ceil, 4) if ceil else None}
    if dist:
        rb = dist["random_block_ceiling"]
        line["roofline"]["random_block_ceiling"] = rb["GBps"]
        line["roofline"]["frac_of_random_block_ceiling"] = dist["frac_random_block_ceiling"]
        line["roofline"]["random_block_ceiling_what"] = rb["what"]
        # the fastest mode measured on the same distinct calls (worklist order,
        # record placement and loop are the caller's choices)
        modes = {k: v for k, v in dist.items() if isinstance(v, dict) and "hbm_GBps_kernel" in v
                 and k != "random_block_ceiling"}
        if modes:
            best = max(modes, key=lambda k: modes[k]["hbm_GBps_kernel"])
            line["roofline"]["best_mode"] = {
                "mode": best, "achieved": modes[best]["hbm_GBps_kernel"],
                "frac": round(modes[best]["hbm_GBps_kernel"] / HBM_PEAK_GBS, 4),
                "kernel_us": modes[best]["kernel_us_p50"],
                "frac_of_random_block_ceiling": round(rb["us"] / modes[best]["kernel_us_p50"], 4)}
            # the fastest mode on the list as given (no caller-side sort):
            # what the library's own flags reach
            own = {k: v for k, v in modes.items() if "sorted" not in k}
            if own:
                b2 = max(own, key=lambda k: own[k]["hbm_GBps_kernel"])
                line["roofline"]["best_mode_unsorted_list"] = {
                    "mode": b2, "achieved": own[b2]["hbm_GBps_kernel"],
                    "frac": round(own[b2]["hbm_GBps_kernel"] / HBM_PEAK_GBS, 4),
                    "kernel_us": own[b2]["kernel_us_p50"],
                    **({"events_cover": own[b2]["events_cover"]} if "events_cover" in own[b2]
                       else {})}
    line["d2d"] = res
    line["parity"] = "bit-exact vs oracle"
    return line


# ---------------------------------------------------------------------------
# Mixed sizes
# ---------------------------------------------------------------------------

def bench_mixed(c: Ctx, args):
    W, K, hiprt = c.W, c.K, c.hiprt
    g = args.max_wgs if args.max_wgs is not None else ONE_WAY_MAX_WGS
    rows = {}
    for n in (16, 256, 4096, 65536):
        wl = W.h2d_mixed(seed=0, n=n)
        r = c.Resident(wl)
        b = wl.batches[0]
        pl = K.kvcopy_plan(*r.addrs[0], b.size)
        k = max(5, min(args.steps * 5, 200 if n <= 256 else args.steps))
        s, _ = c.timed_bracketed(r, [0], [c.sA], k, args.leg_warmup, g)
        _, km = c.timed(r, [0], [c.sA], k, 2, g)
        lat = c.latency(r, 0, g, k=50 if n <= 4096 else 10, w=5)
        c.verify(wl, r, [0], f"mixed {n}")       # before the DMA baselines write the same bytes
        dma = dma_baselines(c, pl, b.nbytes, hiprt.H2D_KIND, reps=2 if n <= 4096 else 1)
        rows[str(n)] = {"bytes": b.nbytes, "merged": int(pl.n_merged), "chunks": int(pl.n_chunks),
                        "GBps": round(gbs(b.nbytes, s), 2), "kernel_us": round(km[0] * 1e3, 2),
                        "kernel_GBps": round(gbs(b.nbytes, km[0] / 1e3), 2), "latency": lat,
                        "dma_baselines": dma}
        log(f"  mixed N={n}: {rows[str(n)]} (bit-exact)")
        r.free()
    cl = c_caller_latency([(f"h2d_mixed_{n}", W.h2d_mixed(seed=0, n=n), g) for n in (16, 256, 4096)])
    for n in (16, 256, 4096):
        rows[str(n)]["latency_c_caller"] = cl.get(f"h2d_mixed_{n}", cl.get("error"))
    log(f"  mixed, C caller: {cl}")
    if args.counter_calibration:
        counter_calibration(c)
    top = rows["65536"]
    line = base_line(args, top["GBps"], "GB/s", top["bytes"] / top["GBps"] / 1e9, {
        "workload": "H2D with mixed sizes (70% in 8-16 KiB, rest 4-8 and 16-28 KiB, 8-byte "
                    "multiples), 25% of descriptors adjacent in both arenas, N = 16 .. 65,536; "
                    "value at N = 65,536",
        "max_wgs": g, "chunk_bytes": K.CHUNK_DEFAULT, "seed": 0})
    line["per_n"] = rows
    line["parity"] = "bit-exact vs oracle"
    return line


# ---------------------------------------------------------------------------
# Kernel or the runtime's copy, per batch shape
# ---------------------------------------------------------------------------

# (descriptors, bytes each): lone small blocks, bursts of 4 KiB blocks, 64 KiB
# blocks, 1 MiB rows, and large single ranges
CROSSOVER_SHAPES = ((1, 4 << 10), (4, 4 << 10), (16, 4 << 10), (16384, 4 << 10), (4, 64 << 10),
                    (1024, 64 << 10), (1, 1 << 20), (64, 1 << 20), (1, 4 << 20), (4, 16 << 20),
                    (1, 64 << 20))


def bench_crossover(c: Ctx, args):
    """Kernel or the runtime's copy, per batch shape.  The vLLM PR #42212
    report ("implementation breakdown") routes batches of fewer than 16
    descriptors, or of descriptors above 28 KiB, to DMA.  Here: shuffled
    blocks of one size between mapped pinned memory and HBM, each direction
    alone; the GPU time between events recorded around one call (median of
    several calls, after 3 untimed ones) for one kvcopy_batch at max_wgs
    (default 8) and for one hipMemcpyAsync per range; every shape checked
    bit-exact against the oracle."""
    W, K, hiprt, torch = c.W, c.K, c.hiprt, c.torch
    if args.no_events:
        print("the crossover workload times calls with HIP events; run it without --no-events",
              file=sys.stderr)
        sys.exit(2)
    g = args.max_wgs if args.max_wgs is not None else 8
    st = c.sA

    def median_ms(fn, reps):
        out = []
        for i in range(reps + 3):
            e0, e1 = hiprt.Event(), hiprt.Event()
            e0.record(st)
            fn()
            e1.record(st)
            ms = e0.elapsed_ms(e1)
            if i >= 3:
                out.append(ms)
        return statistics.median(out)

    rows, wins = {}, 0
    for n, size in CROSSOVER_SHAPES:
        for dname in ("h2d", "d2h"):
            wl = W.kv_blocks(seed=0, directions=dname, n=n, pool_blocks=n, block=size)
            r = c.Resident(wl)
            nbytes = wl.batches[0].nbytes
            reps = 20 if n <= 64 else 5
            kern = median_ms(lambda: r.submit(0, g, st), reps)
            r.fill()
            r.submit(0, g, st)
            torch.cuda.synchronize()
            c.verify(wl, r, [0], f"crossover {n} x {size} {dname}")
            pl = K.kvcopy_plan(*r.addrs[0], wl.batches[0].size)
            kind = hiprt.H2D_KIND if dname == "h2d" else hiprt.D2H_KIND
            ranges = list(zip(pl.src.tolist(), pl.dst.tolist(), pl.size.tolist()))

            def per_range():
                for s_, d_, z_ in ranges:
                    hiprt.memcpy_async(d_, s_, z_, kind, st)

            rt = median_ms(per_range, reps)
            key = f"{n}x{size}/{dname}"
            rows[key] = {"kernel_us": round(kern * 1e3, 2), "kernel_GBps": round(gbs(nbytes, kern / 1e3), 3),
                         "runtime_copy_us": round(rt * 1e3, 2),
                         "runtime_copy_GBps": round(gbs(nbytes, rt / 1e3), 3),
                         "runtime_copies": len(ranges)}
            wins += kern <= rt
            log(f"  crossover {key}: {rows[key]}")
            r.free()
    # Both calls above are issued from Python, where kvcopy_batch carries a few
    # microseconds more marshalling (three arrays) than one hipMemcpyAsync
    # call; for the small batches the same kernel calls are also timed from C
    # (the C-caller tool: events around the call, host time inside it).
    named = [(f"{n}x{size}_{dname}", W.kv_blocks(seed=0, directions=dname, n=n, pool_blocks=n,
                                                block=size), g)
             for n, size in CROSSOVER_SHAPES if n <= 16 and size <= (64 << 10)
             for dname in ("h2d", "d2h")]
    cl = c_caller_latency(named + [(f"{nm}_runtime", wl_, g_, RUNTIME_COPY_FLAG)
                                   for nm, wl_, g_ in named])
    for key, row in rows.items():
        crow = cl.get(key.replace("/", "_"))
        rrow = cl.get(key.replace("/", "_") + "_runtime")
        if crow:
            row["kernel_call_gpu_us_from_c"] = crow.get("gpu_us_p50")
            row["kernel_call_host_us_from_c"] = crow.get("host_us_p50")
        if rrow:
            row["runtime_copy_gpu_us_from_c"] = rrow.get("gpu_us_p50")
    if "error" in cl:
        log(f"  crossover, C caller: {cl['error']}")
    line = base_line(args, wins, "shapes", 0.0, {
        "workload": "one kvcopy_batch against one hipMemcpyAsync per range, shuffled blocks "
                    "between mapped pinned memory and HBM, each direction alone, "
                    f"{len(CROSSOVER_SHAPES)} shapes from 1 x 4 KiB to 1 x 64 MiB; value = shapes "
                    "(of both directions) where the kernel call takes no longer",
        "max_wgs": g, "chunk_bytes": K.CHUNK_DEFAULT, "seed": 0}, dtype="u8")
    line["shapes"] = rows
    line["parity"] = "bit-exact vs oracle"
    return line


# ---------------------------------------------------------------------------
# MoE expert gather
# ---------------------------------------------------------------------------

def call_us(c: Ctx, submit, stream):
    """Microseconds of one call: GPU time between events recorded around it,
    or, with --no-events (profiler runs, which make no event calls), wall
    time from a synchronised stream to the call's completion."""
    hiprt = c.hiprt
    if c.args.no_events:
        hiprt.stream_sync(stream)
        t0 = time.perf_counter()
        submit()
        hiprt.stream_sync(stream)
        return (time.perf_counter() - t0) * 1e6
    e0, e1 = hiprt.Event(), hiprt.Event()
    e0.record(stream)
    submit()
    e1.record(stream)
    return e0.elapsed_ms(e1) * 1e3


def bench_moe(c: Ctx, args):
    W, K, hiprt = c.W, c.K, c.hiprt
    calls = 100
    wl = W.moe_gather(seed=0, calls=calls)
    r = c.Resident(wl)
    out = {}
    # byte-balanced: 16 KiB chunks dealt to all wavefronts; unbalanced: one
    # wavefront per row (chunk = 1 MiB), the descriptor-granular work split
    for name, chunk in (("byte_balanced_16KiB", 0), ("one_wave_per_row", K.CHUNK_MAX)):
        for g in (8, 32, 128, 0):
            t_us, sizes = [], []
            with no_gc():
                for i in range(calls):
                    t_us.append(call_us(c, lambda: r.submit(i, g, c.sA, chunk_bytes=chunk), c.sA))
                    sizes.append(wl.batches[i].nbytes)
            rates = [gbs(z, t / 1e6) for z, t in zip(sizes, t_us)]
            out[f"{name}/max_wgs={g}"] = {
                "call_us_p50": round(pct(t_us, 50), 1), "call_us_p99": round(pct(t_us, 99), 1),
                "GBps_p50": round(pct(rates, 50), 2), "GBps_total": round(gbs(sum(sizes), sum(t_us) / 1e6), 2)}
            log(f"  moe {name} max_wgs={g}: {out[f'{name}/max_wgs={g}']}")
    c.verify(wl, r, list(range(calls)), "moe")     # every call wrote its slots; the last writes win
    r.free()
    # Context row: 1-8 missed experts per call (one layer's top-8 misses).
    small = W.moe_gather(seed=1, calls=calls, misses=(1, 8))
    r = c.Resident(small)
    t_us, sizes = [], []
    with no_gc():
        for i in range(calls):
            t_us.append(call_us(c, lambda: r.submit(i, 32, c.sA), c.sA))
            sizes.append(small.batches[i].nbytes)
    c.verify(small, r, list(range(calls)), "moe 1-8 misses")
    r.free()
    out["context_1_to_8_misses/max_wgs=32"] = {
        "call_us_p50": round(pct(t_us, 50), 1), "call_us_p99": round(pct(t_us, 99), 1),
        "GBps_total": round(gbs(sum(sizes), sum(t_us) / 1e6), 2)}
    log(f"  moe 1-8 misses: {out['context_1_to_8_misses/max_wgs=32']}")
    # Device-resident miss lists, one HIP graph per call (kvcopy_batch_device):
    # the decode-side form in which a router kernel leaves the list on the GPU.
    for name, misses in (() if args.no_events else
                         (("device_graph_26_to_39_misses", (26, 39)),
                          ("device_graph_1_to_8_misses", (1, 8)))):
        out[f"{name}/max_wgs=32"] = moe_device_graph(c, W.moe_gather(seed=2, calls=calls,
                                                                    misses=misses), 32)
        log(f"  moe {name}: {out[f'{name}/max_wgs=32']}")
    best = max((v["GBps_total"], k) for k, v in out.items() if k.startswith("byte_balanced"))
    line = base_line(args, best[0], "GB/s", 0.0, {
        "workload": "MoE expert gather: 100 seeded calls, each 26-39 experts x 6 bank rows "
                    "(1 MiB, 64 KiB, 4 KiB, 512 KiB, 32 KiB, 4 KiB) from pinned host banks into "
                    "random slots of a 3,164-slot device cache; one call per step",
        "best": best[1], "seed": 0})
    line["ms_per_step"] = round(out[best[1]]["call_us_p50"] / 1e3, 4)
    line["steps"] = calls
    line["per_setting"] = out
    line["parity"] = "bit-exact vs oracle"
    if args.counter_calibration:
        counter_calibration(c)
    return line


def moe_device_graph(c: Ctx, wl, max_wgs):
    """Each call's descriptor list and count are placed in device memory
    beforehand, and one HIP graph per call captures kvcopy_batch_device on
    them; the graphs are then replayed in order on one stream, each bracketed
    by events.  Checked bit-exact against the oracle at the end."""
    np, torch, K, hiprt = c.np, c.torch, c.K, c.hiprt
    r = c.Resident(wl)
    calls = len(wl.batches)
    max_n = max(b.n for b in wl.batches)
    lists = []
    for i, b in enumerate(wl.batches):
        s_, d_ = r.addrs[i]
        t = torch.zeros((3, max_n), dtype=torch.int64, device=c.dev)
        for row, a in enumerate((s_, d_, b.size)):
            t[row, :b.n].copy_(torch.from_numpy(np.ascontiguousarray(a).view(np.int64)))
        lists.append((t, torch.tensor([b.n], dtype=torch.int64, device=c.dev)))
    ws = torch.empty(K.kvcopy_device_workspace_bytes(max_n) + 256, dtype=torch.uint8, device=c.dev)
    base = (ws.data_ptr() + 255) // 256 * 256
    st = c.sA

    def call(i):
        t, n = lists[i]
        K.kvcopy_batch_device(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), n.data_ptr(),
                              max_n, K.H2D, max_wgs, base, stream=st.cuda_stream)

    with torch.cuda.stream(st):
        call(0)                      # warm-up outside any graph
    torch.cuda.synchronize()
    graphs = []
    for i in range(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            call(i)
        graphs.append(g)
    torch.cuda.synchronize()
    r.fill()
    t_us = []
    with no_gc(), torch.cuda.stream(st):
        for i in range(calls):
            e0, e1 = hiprt.Event(), hiprt.Event()
            e0.record(st)
            graphs[i].replay()
            e1.record(st)
            t_us.append(e0.elapsed_ms(e1) * 1e3)
    torch.cuda.synchronize()
    status = int(ws[base - ws.data_ptr():base - ws.data_ptr() + 8].cpu().numpy().view(np.uint64)[0])
    if status != 0:
        log(f"DEVICE BATCH STATUS {status}")
        sys.exit(3)
    c.verify(wl, r, list(range(calls)), "moe device graphs")
    sizes = [b.nbytes for b in wl.batches]
    del graphs
    r.free()
    return {"call_us_p50": round(pct(t_us, 50), 1), "call_us_p99": round(pct(t_us, 99), 1),
            "GBps_total": round(gbs(sum(sizes), sum(t_us) / 1e6), 2), "calls": calls}


# ---------------------------------------------------------------------------
# Interference: decode loop vs bidirectional bursts
# ---------------------------------------------------------------------------

def parse_mode(mode):
    """(kind, cap, options) of an interference mode.  Modes: "none" (no
    transfer), "direct" (one hipMemcpyAsync per fragment), an integer cap G
    (both directions on two streams at G workgroups each; 0 = full grid),
    "G/sc1" or "G/nt" (the same with the store form forced on both kernels),
    "tail" (two streams with KVCOPY_F_TAIL_BOUNDED; "tail/nt" with nt stores),
    "duty:ON:PERIOD:G" (the same with time-sliced issue, ON and PERIOD in
    microseconds), "pair:G" and "pair:G/nt" (both lists in one launch),
    "pipe:G" (the pipelined loop forced), "job:N" (paced pieces of N
    descriptors), "h2d:G" and "d2h:G" (one direction alone), "cumask:N" (two
    streams at the full grid on the first N compute units)."""
    if isinstance(mode, int):
        return "streams", mode, {}
    m = str(mode)
    if m in ("none", "direct"):
        return m, 0, {}
    opt = {}
    if "/" in m:
        m, store = m.split("/", 1)
        if store not in ("sc1", "nt"):
            raise ValueError(f"unknown store form in interference mode {mode!r}")
        opt["store"] = store
    if m.isdigit():
        return "streams", int(m), opt
    head, _, rest = m.partition(":")
    if head == "tail":
        opt["tail"] = True
        return "streams", 0, opt
    if head == "duty":
        on, per, cap = rest.split(":")
        opt["duty"] = (int(round(float(on) * 1000)), int(round(float(per) * 1000)))
        return "streams", int(cap), opt
    if head in ("pair", "pipe", "job", "h2d", "d2h", "cumask") and rest.isdigit():
        return head, int(rest), opt
    raise ValueError(f"unknown interference mode {mode!r}")


def bench_interference(c: Ctx, args):
    torch, W, K, hiprt = c.torch, c.W, c.K, c.hiprt
    from block_copy_amd.decode_load import AluChain, Chain
    d_model, d_ff, n_gemv = 2560, 9728, 36
    if args.decode_kind == "alu":
        # the ALU-only stand-in: 36 kernels that touch memory only in their
        # last store (one per workgroup)
        chain = AluChain(torch.zeros(1024, dtype=torch.float32, device=c.dev), n=n_gemv,
                         grid=args.alu_grid, iters=args.alu_iters)
        wbytes = 0
        decode_what = (f"decode stand-in of {n_gemv} ALU-only kernels ({args.alu_grid} workgroups "
                       f"x 256 threads, {args.alu_iters} dependent FMAs per thread, one store per "
                       "workgroup)")
    else:
        g = torch.Generator(device=c.dev)
        g.manual_seed(0)
        weights, acts = [], [torch.randn(d_model, generator=g, device=c.dev).to(torch.bfloat16)]
        for i in range(n_gemv):
            shape = (d_ff, d_model) if i % 2 == 0 else (d_model, d_ff)
            weights.append((torch.randn(shape, generator=g, device=c.dev) * 0.02).to(torch.bfloat16))
            acts.append(torch.empty(shape[0], dtype=torch.bfloat16, device=c.dev))
        chain = Chain(weights, acts)
        wbytes = sum(w.numel() * 2 for w in weights)
        decode_what = (f"decode loop of {n_gemv} bf16 GEMVs ({d_ff}x{d_model} and {d_model}x{d_ff}, "
                       f"{wbytes / 1e9:.2f} GB of distinct weights per step)")
    try:                               # the decode stream: a hardware queue of its own
        dq = hiprt.QueueStreams(1, torch.cuda.get_device_properties(c.dev).multi_processor_count)
        sD = dq.streams[0]
    except RuntimeError as e:
        log(f"  dedicated-queue decode stream unavailable ({e}); using a torch stream")
        sD = torch.cuda.Stream()
    wl = W.kv_blocks(seed=0, directions="both")
    r = c.Resident(wl)
    period = 0.050
    steps, warm = args.decode_steps, 32

    masked = {}

    def run(mode):
        stop = threading.Event()
        moved = [0]
        bursts = [0]
        sa, sb = c.sA, c.sB
        if isinstance(mode, str) and mode.startswith("cumask"):
            # copy streams restricted to the first N compute units
            ncu = int(mode.split(":")[1])
            if ncu not in masked:
                masked[ncu] = (hiprt.CUMaskStream(range(ncu)), hiprt.CUMaskStream(range(ncu)))
            sa, sb = masked[ncu]
            mode = 0          # the full grid, on the masked compute units

        kind, g, opt = parse_mode(mode)
        copy_kw = {}
        if opt.get("store"):
            copy_kw["flags"] = K.F_STORE_SC1 if opt["store"] == "sc1" else K.F_STORE_NT
        if opt.get("tail"):
            copy_kw["flags"] = copy_kw.get("flags", 0) | K.F_TAIL_BOUNDED
        if opt.get("duty"):
            copy_kw["duty_on_ns"], copy_kw["duty_period_ns"] = opt["duty"]

        def transfer():
            nxt = time.perf_counter()
            while not stop.is_set():
                if kind == "direct":
                    for j, kd, st in ((0, hiprt.H2D_KIND, c.sA), (1, hiprt.D2H_KIND, c.sB)):
                        b = wl.batches[j]
                        s_, d_ = r.addrs[j]
                        for x, y, z in zip(s_.tolist(), d_.tolist(), b.size.tolist()):
                            hiprt.memcpy_async(y, x, z, kd, st)
                elif kind == "job":
                    # paced pieces: the next piece goes only after the previous completed
                    jobs = [K.kvcopy_job_create(*r.addrs[j], wl.batches[j].size, wl.batches[j].dir,
                                                0, g, st.cuda_stream)
                            for j, st in ((0, c.sA), (1, c.sB))]
                    pending = list(jobs)
                    while pending:
                        pending = [jb for jb in pending if not K.kvcopy_job_poll(jb)]
                        if pending:
                            time.sleep(20e-6)      # yield the worker while a piece runs
                    for jb in jobs:
                        K.kvcopy_job_destroy(jb)
                elif kind == "pair":
                    # both lists in one launch (kvcopy_batch_pair) on one stream
                    (s0, d0), (s1, d1) = r.addrs[0], r.addrs[1]
                    K.kvcopy_batch_pair(s0, d0, wl.batches[0].size, s1, d1, wl.batches[1].size, g,
                                        sa.cuda_stream,
                                        flags=K.F_STORE_NT if opt.get("store") == "nt" else 0)
                elif kind == "pipe":
                    # the pipelined loop forced at a small cap
                    r.submit(0, g, sa, flags=K.F_PIPELINE)
                    r.submit(1, g, sb, flags=K.F_PIPELINE)
                elif kind in ("h2d", "d2h"):
                    # one direction alone
                    r.submit(0 if kind == "h2d" else 1, g, sa, **copy_kw)
                else:                               # two streams at cap g
                    r.submit(0, g, sa, **copy_kw)
                    r.submit(1, g, sb, **copy_kw)
                hiprt.stream_sync(sa)
                hiprt.stream_sync(sb)
                moved[0] += wl.batches[0 if kind == "h2d" else 1].nbytes if kind in ("h2d", "d2h") \
                    else wl.nbytes
                bursts[0] += 1
                nxt += period
                delay = nxt - time.perf_counter()
                if delay > 0:
                    stop.wait(delay)
                else:
                    nxt = time.perf_counter()

        th = None
        for _ in range(warm):
            chain.run(sD)
        hiprt.stream_sync(sD)
        t_start = time.perf_counter()
        if mode != "none":
            th = threading.Thread(target=transfer, daemon=True)
            th.start()
        gpu_ms, wall_ms = [], []
        # --no-events (profiler runs): no event pairs; the step's wall time
        # (launches + stream sync) stands in for its GPU time
        evs = [(None, None) if args.no_events else (hiprt.Event(), hiprt.Event())
               for _ in range(steps)]
        with no_gc():
            for e0, e1 in evs:
                t0 = time.perf_counter()
                if e0 is not None:
                    e0.record(sD)
                chain.run(sD)
                if e1 is not None:
                    e1.record(sD)
                hiprt.stream_sync(sD)
                wall_ms.append((time.perf_counter() - t0) * 1e3)
        gpu_ms = wall_ms if args.no_events else [e0.elapsed_ms(e1) for e0, e1 in evs]
        dur = time.perf_counter() - t_start
        if th is not None:
            stop.set()
            th.join()
        return gpu_ms, wall_ms, moved[0] / dur, bursts[0]

    modes = ["none", "direct", 1, 8, 32, 128, 0, "8/sc1", "128/sc1", "8/nt", "h2d:8", "d2h:8",
             "h2d:128", "d2h:128", "pipe:4", "job:2048", "cumask:8", "pair:8", "pair:16",
             "pair:64", "pair:8/nt", "pair:16/nt", "duty:2:20:8", "duty:2:20:4", "duty:2:20:4/sc1",
             "duty:2:40:4/sc1", "duty:2:10:128", "tail"]
    if args.modes:     # a subset or other modes; "none" (the baseline) always runs
        pick = [m for m in args.modes.split(",") if m]
        try:
            for m in pick:
                parse_mode(m)
        except ValueError as e:
            print(f"{e}; see parse_mode for the forms", file=sys.stderr)
            sys.exit(2)
        modes = ["none"] + [int(m) if m.isdigit() else m for m in pick if m != "none"]
    results = {str(m): {"gpu": [], "wall": [], "rate": [], "bursts": 0} for m in modes}
    for rep in range(args.decode_runs):
        order = modes[rep % len(modes):] + modes[:rep % len(modes)]
        for m in order:
            gms, wms, rate, nb = run(m)
            rr = results[str(m)]
            rr["gpu"].append(gms)
            rr["wall"].append(wms)
            rr["rate"].append(rate)
            rr["bursts"] += nb
            log(f"  interference run {rep} mode {m}: p50 {pct(gms, 50):.3f} p99 {pct(gms, 99):.3f} "
                f"max {max(gms):.3f} ms (GPU), wall p99 {pct(wms, 99):.3f} ms, "
                f"{rate / 2**30:.3f} GiB/s, {nb} bursts")
    hiprt.stream_sync(c.sA)
    hiprt.stream_sync(c.sB)
    c.verify(wl, r, [0, 1], "interference bursts")
    r.free()
    for pair_ in masked.values():
        for st in pair_:
            st.destroy()
    if isinstance(sD, torch.cuda.ExternalStream):
        dq.destroy()
    table = {}
    for m, rr in results.items():
        def agg(key, q):
            return round(statistics.mean(pct(x, q) for x in rr[key]), 4)
        table[m] = {"gpu_ms_mean": round(statistics.mean(statistics.mean(x) for x in rr["gpu"]), 4),
                    "gpu_ms_p50": agg("gpu", 50), "gpu_ms_p99": agg("gpu", 99),
                    "gpu_ms_max": round(max(max(x) for x in rr["gpu"]), 4),
                    "wall_ms_p50": agg("wall", 50), "wall_ms_p99": agg("wall", 99),
                    "wall_ms_max": round(max(max(x) for x in rr["wall"]), 4),
                    "transfer_GiBps": round(statistics.mean(rr["rate"]) / 2**30, 3),
                    "bursts": rr["bursts"]}
    base = table["none"]["gpu_ms_p99"]
    for m in table:
        table[m]["p99_vs_none"] = round(table[m]["gpu_ms_p99"] / base - 1, 4)
        # decode time lost per burst: the extra mean step time over all timed
        # steps, shared out over the bursts that ran meanwhile (p99 and max
        # show how the loss is spread; this shows how large it is)
        n_steps = sum(len(x) for x in results[m]["gpu"])
        if table[m]["bursts"]:
            table[m]["decode_ms_lost_per_burst"] = round(
                (table[m]["gpu_ms_mean"] - table["none"]["gpu_ms_mean"]) * n_steps
                / table[m]["bursts"], 3)
    # the line's value: the tail-bounded preset (the library's setting for
    # copies beside latency-sensitive kernels) when it ran, else 32 per stream
    headline_mode = next((m for m in ("tail", "32") if m in table),
                         next((m for m in table if m != "none"), "none"))
    line = base_line(args, table[headline_mode]["gpu_ms_p99"], "ms", table["none"]["gpu_ms_mean"] / 1e3, {
        "workload": f"{decode_what} while a bidirectional "
                    "burst (16,384 x 4 KiB H2D + 16,384 x 4 KiB D2H) starts every 50 ms; value = "
                    f"decode step p99 ({'wall' if args.no_events else 'GPU'} time) in mode "
                    f"{headline_mode} (an integer mode is max_wgs on two streams; tail is "
                    "KVCOPY_F_TAIL_BOUNDED on two streams)",
        "decode_steps_per_run": steps, "runs_per_mode": args.decode_runs, "seed": 0},
        dtype="bf16", higher=False)
    line["modes"] = table
    line["parity"] = "bit-exact vs oracle (last burst)"
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 600 steps of the headline burst time about 0.9 s.  Measured on MI355X,
    # the rate of two copy kernels on two streams varies over time: 20-step
    # windows at 68-81 GB/s against 85-88 in between, in stretches of up to
    # a few hundred ms, so a 0.15 s timed region read 71-82 GB/s in 3 of 8
    # processes; a longer one averages over those stretches as a long run does
    ap.add_argument("--steps", type=int, default=600)
    # The workload's own step warms up for 700 steps (about a second of the
    # headline burst): measured on MI355X, the first second of bidirectional
    # traffic in a process runs a few percent slower (two 600-step runs back
    # to back: 84.4-87.0 GB/s, then 88.0-88.2).  Secondary legs warm up for
    # at most 100 of their own steps (args.leg_warmup).
    ap.add_argument("--warmup", type=int, default=700)
    ap.add_argument("--max-wgs", type=parse_wgs, default=None,
                    help=f"workgroup cap (kv: {DEFAULT_MAX_WGS} per stream; mixed: {ONE_WAY_MAX_WGS}; "
                         "pair: KVCOPY_WGS_AUTO); "
                         "kv only: H2D,D2H for a cap per direction")
    ap.add_argument("--copy-cus", default="halves", choices=["all", "halves"],
                    help="kv: CU masks of the headline's two copy streams, disjoint halves "
                         "(default; each XCD keeps CUs for both) or every CU")
    ap.add_argument("--workload", default="kv", choices=["kv", "pair", "d2d", "mixed", "moe",
                                                         "interference", "crossover"])
    ap.add_argument("--sweep", action="store_true", help="also sweep max_wgs per direction (stderr)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the cpu_baseline sample")
    ap.add_argument("--skip-extras", action="store_true",
                    help="only the headline workload (for profiling runs)")
    ap.add_argument("--no-events", action="store_true",
                    help="make no HIP event calls (profiler runs): kernels are not bracketed, "
                         "the kernel time is taken as the step time, and the two directions "
                         "of a step are not joined")
    ap.add_argument("--counter-calibration", action="store_true",
                    help="also run a plain 64 MiB elementwise copy kernel 5 times, whose "
                         "known traffic scales the PMC byte counters")
    ap.add_argument("--desc-upload", action="store_true",
                    help="upload worklists to device memory before each kernel (KVCOPY_F_DESC_UPLOAD) "
                         "instead of reading them in place from pinned staging")
    ap.add_argument("--flags", type=lambda x: int(x, 0), default=0,
                    help="kvcopy_batch_ex flags added to every call of the timed steps "
                         "(measurement only; e.g. 0x800 = KVCOPY_F_WG_PER_CHUNK)")
    ap.add_argument("--store", default="auto",
                    help="store form of the copy kernels in the timed steps (KVCOPY_F_STORE_SC1 / "
                         "KVCOPY_F_STORE_NT): auto (the library's choice), sc1, nt, or per "
                         "direction as h2d:sc1,d2h:nt")
    ap.add_argument("--decode-steps", type=int, default=1536)
    ap.add_argument("--decode-runs", type=int, default=3)
    ap.add_argument("--modes", default="",
                    help="interference: comma-separated modes to run (default: a fixed list; "
                         "see parse_mode)")
    ap.add_argument("--decode-kind", default="gemv", choices=["gemv", "alu"],
                    help="interference: the bf16 GEMV chain, or the ALU-only stand-in")
    ap.add_argument("--alu-iters", type=int, default=4096,
                    help="interference with --decode-kind alu: dependent FMAs per thread")
    ap.add_argument("--alu-grid", type=int, default=1024,
                    help="interference with --decode-kind alu: workgroups per kernel")
    args = ap.parse_args()
    args.leg_warmup = min(args.warmup, 100)
    if isinstance(args.max_wgs, list) and args.workload != "kv":
        print("a cap per direction (--max-wgs H2D,D2H) applies to --workload kv only",
              file=sys.stderr)
        sys.exit(2)
    try:
        store_forms(args.store)
    except ValueError as e:
        print(e, file=sys.stderr)
        sys.exit(2)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the copy path has no multi-GPU step "
              "(each GPU would run the same kernel on its own share of the descriptors); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    c = Ctx(args)
    fn = {"kv": bench_kv, "pair": bench_pair, "d2d": bench_d2d, "mixed": bench_mixed, "moe": bench_moe,
          "interference": bench_interference, "crossover": bench_crossover}[args.workload]
    line = fn(c, args)
    print(json.dumps(line), flush=True)
    c.close()


if __name__ == "__main__":
    main()
