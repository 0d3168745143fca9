#!/usr/bin/env python3
"""Benchmark of the batched descriptor copy on one MI355X.

Workload (the headline): bidirectional bursts of 16,384 shuffled 4 KiB
descriptors host->device plus 16,384 shuffled 4 KiB descriptors
device->host, submitted concurrently on two streams against a 65,536-block
(256 MiB) device KV pool and mapped pinned host buffers (64 MiB per
direction).  One step = one such burst through the whole path: validate,
coalesce and chunk on the host, one worklist upload and one kernel launch
per direction.  ``value`` is payload bytes moved per second (GB/s = 1e9 B/s)
over the timed steps, inputs resident before the timed region.

Also reported, each in the same run: each direction alone; the contiguous
hipMemcpyAsync ceilings of the host link (the practical peak); one
hipMemcpyAsync per fragment (the baseline the method replaces); the D2D
gather of 1,024 x 4 KiB blocks and a scaled D2D variant against HBM; and
the CPU oracle timed on the host cores on a bounded sample.  Every GPU result
is checked bit-exact against the oracle before the line is printed.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--max-wgs G]
Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s for batched 4–16 KiB descriptor copies (H2D/D2H/D2D), % of link/HBM peak"
PCIE_PEAK_GBS = 64.0      # PCIe 5.0 x16, per direction (MI355X host interface)
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
# Workgroup cap of the headline: with H2D and D2H running together, a few
# dozen workgroups per direction keep enough bytes in flight to fill the
# link; the full grid oversubscribes it (see the max_wgs sweep, --sweep).
DEFAULT_MAX_WGS = 32
KERNEL_NAMES = {0: "kvcopy_h2d_kernel", 1: "kvcopy_d2h_kernel"}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_kv_bidirectional.json")
KERNEL_SOURCE = os.path.join(ROOT, "block_copy_amd", "csrc", "kvcopy_kernel.hip")


def kernel_source_hash():
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel):
    """HBM/host bytes per launch of `kernel` from the committed PMC summary,
    or None if there is none or the kernel source changed since it was taken."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != kernel_source_hash():
        return None
    k = c.get("kernels", {}).get(kernel)
    if not k:
        return None
    return {"fetch_bytes": k["fetch_bytes_per_dispatch_scaled"],
            "write_bytes": k["write_bytes_per_dispatch_scaled"],
            "source": os.path.relpath(COUNTERS_FILE, ROOT)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gbs(nbytes, seconds):
    return nbytes / seconds / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--max-wgs", type=int, default=DEFAULT_MAX_WGS)
    ap.add_argument("--sweep", action="store_true", help="also sweep max_wgs per direction (stderr)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the cpu_baseline sample")
    ap.add_argument("--skip-extras", action="store_true",
                    help="only the headline workload (for profiling runs)")
    ap.add_argument("--no-events", action="store_true",
                    help="do not bracket kernels with HIP events (profiler runs); the kernel "
                         "time is then taken as the step time")
    ap.add_argument("--counter-calibration", action="store_true",
                    help="also run a plain 64 MiB elementwise copy kernel 5 times, whose "
                         "known traffic scales the PMC byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the copy path has no multi-GPU step "
              "(see the sharding note in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from block_copy_amd import hiprt
    from block_copy_amd import kvcopy as K
    from block_copy_amd.harness import Resident

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({props.gcnArchName}), {props.multi_processor_count} CUs")

    # ---------------- headline: bidirectional 16,384 x 4 KiB per direction ---------------
    wl = W.kv_blocks(seed=0, directions="both")
    res = Resident(wl)
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    step_bytes = wl.nbytes
    n_desc = sum(b.n for b in wl.batches)

    def run_steps(r, batch_ids, streams, k, max_wgs, events=None):
        for i in range(k):
            for j, (bi, st) in enumerate(zip(batch_ids, streams)):
                kw = {}
                if events is not None:
                    kw = dict(kernel_begin=events[i][j][0].h, kernel_end=events[i][j][1].h)
                r.submit(bi, max_wgs, st, **kw)

    def timed(r, batch_ids, streams, k, w, max_wgs, with_events=True):
        """Seconds per step over k timed steps (after w warm-up steps), and the
        mean kernel-only duration (ms) of each batch from HIP events."""
        run_steps(r, batch_ids, streams, w, max_wgs)
        torch.cuda.synchronize()
        evs = [[(hiprt.Event(), hiprt.Event()) for _ in batch_ids] for _ in range(k)] \
            if with_events else None
        t0 = time.perf_counter()
        run_steps(r, batch_ids, streams, k, max_wgs, evs)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kern = None
        if evs:
            kern = [statistics.mean(evs[i][j][0].elapsed_ms(evs[i][j][1]) for i in range(k))
                    for j in range(len(batch_ids))]
        return (t1 - t0) / k, kern

    max_wgs = args.max_wgs
    log(f"headline: {n_desc} descriptors, {step_bytes} B per step, max_wgs={max_wgs}")
    step_s, kern_ms = timed(res, [0, 1], [sA, sB], args.steps, args.warmup, max_wgs,
                            with_events=not args.no_events)
    if kern_ms is None:
        kern_ms = [step_s * 1e3, step_s * 1e3]
    value = gbs(step_bytes, step_s)
    log(f"  bidirectional: {step_s * 1e3:.3f} ms/step, {value:.2f} GB/s; kernel ms {kern_ms}")

    # worklist bytes the kernel reads per launch: one 24-byte record per chunk
    plan = [K.kvcopy_plan(*res.addrs[j], wl.batches[j].size) for j in range(2)]
    meta = [p.n_chunks * 24 for p in plan]
    algo = [wl.batches[j].nbytes + meta[j] for j in range(2)]
    ach = [gbs(algo[j], kern_ms[j] / 1e3) for j in range(2)]

    extras = {}
    if args.sweep:
        sweep = {}
        for name, ids, sts in (("h2d", [0], [sA]), ("d2h", [1], [sA]), ("both", [0, 1], [sA, sB])):
            for g in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 0):
                s_, km = timed(res, ids, sts, max(3, args.steps // 2), 2, g)
                nbytes = sum(wl.batches[i].nbytes for i in ids)
                sweep[f"{name}/{g}"] = round(gbs(nbytes, s_), 2)
                log(f"  sweep {name} max_wgs={g}: {gbs(nbytes, s_):.2f} GB/s, kernel ms "
                    f"{[round(x, 3) for x in km]}")
        extras["max_wgs_sweep_GBps"] = sweep
    if not args.skip_extras:
        # each direction alone
        alone = {}
        for j, name in ((0, "h2d"), (1, "d2h")):
            s, km = timed(res, [j], [sA], args.steps, args.warmup, max_wgs)   # extras only
            alone[name] = {"GBps": round(gbs(wl.batches[j].nbytes, s), 3),
                           "ms_per_call": round(s * 1e3, 4), "kernel_ms": round(km[0], 4)}
            log(f"  {name} alone: {alone[name]}")
        extras["per_direction_alone"] = alone

        # contiguous ceilings: 64 MiB from/to mapped pinned memory, separate buffers
        nb = 64 * W.MIB
        hsrc = K.HostBuffer(nb)
        hdst = K.HostBuffer(nb)
        hsrc.array[:] = 7
        dbuf = torch.empty(2 * nb, dtype=torch.uint8, device=dev)

        def ceiling(kinds, reps=10):
            streams = [sA, sB]
            times = []
            for r in range(reps + 2):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for i, kind in enumerate(kinds):
                    if kind == "h2d":
                        hiprt.memcpy_async(dbuf.data_ptr(), hsrc.ptr, nb, hiprt.H2D_KIND, streams[i])
                    else:
                        hiprt.memcpy_async(hdst.ptr, dbuf.data_ptr() + nb, nb, hiprt.D2H_KIND, streams[i])
                torch.cuda.synchronize()
                if r >= 2:
                    times.append(time.perf_counter() - t0)
            return gbs(nb * len(kinds), statistics.median(times))

        ceil = {"h2d": ceiling(["h2d"]), "d2h": ceiling(["d2h"]), "both": ceiling(["h2d", "d2h"])}
        extras["contiguous_memcpy_ceiling_GBps"] = {k: round(v, 3) for k, v in ceil.items()}
        log(f"  contiguous ceilings: {extras['contiguous_memcpy_ceiling_GBps']}")

        # one hipMemcpyAsync per fragment (after coalescing), one stream
        frag = {}
        for j, name, kind in ((0, "h2d", hiprt.H2D_KIND), (1, "d2h", hiprt.D2H_KIND)):
            p = plan[j]
            reps = 2
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                for s_, d_, z_ in zip(p.src.tolist(), p.dst.tolist(), p.size.tolist()):
                    hiprt.memcpy_async(d_, s_, z_, kind, sA)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / reps
            frag[name] = {"GBps": round(gbs(wl.batches[j].nbytes, dt), 3),
                          "ms_per_call": round(dt * 1e3, 3), "copies": int(p.n_merged)}
            log(f"  per-fragment hipMemcpyAsync {name}: {frag[name]}")
        extras["per_fragment_memcpy"] = frag
        del dbuf
        hsrc.free()
        hdst.free()

    if args.counter_calibration:
        a = torch.arange(16 * W.MIB, dtype=torch.int32, device=dev)   # 64 MiB
        b = torch.empty_like(a)
        for _ in range(5):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    # ---------------- verification of the headline workload ----------------
    torch.cuda.synchronize()
    final = {i: res.image(i) for i in (0, 2)}      # device pool, host D2H destination

    # ---------------- cpu_baseline: the oracle on host images of the same step --------------
    import oracle
    imgs = [a.host_image().copy() if a.fill == "random" else
            np.full(a.nbytes, a.sentinel, np.uint8) for a in wl.arenas]
    src_snap = {0: imgs[0].copy(), 1: imgs[1]}
    bases = res.bases

    def oracle_step():
        moved = 0
        for j in range(2):
            b = wl.batches[j]
            s, d = res.addrs[j]
            si, di = int(b.src_arena[0]), int(b.dst_arena[0])
            moved += oracle.copy(s, d, b.size, [(bases[si], src_snap[si])], [(bases[di], imgs[di])])
        return moved

    reps, moved, t0 = 0, 0, time.perf_counter()
    while True:
        moved += oracle_step()
        reps += 1
        if time.perf_counter() - t0 >= args.cpu_seconds and reps >= 3:
            break
    cpu_s = time.perf_counter() - t0
    cpu_gbs = gbs(moved, cpu_s)
    log(f"  cpu oracle: {reps} steps in {cpu_s:.2f} s = {cpu_gbs:.2f} GB/s (1 thread)")
    for i in (0, 2):
        if not np.array_equal(final[i], imgs[i]):
            bad = int(np.flatnonzero(final[i] != imgs[i])[0])
            log(f"PARITY FAILURE in arena {wl.arenas[i].name} at byte {bad}")
            sys.exit(3)
    log("  parity: bit-exact against the oracle")
    res.free()

    # ---------------- D2D: 1,024 x 4 KiB, and a scaled variant -------------------------------
    if not args.skip_extras:
        d2d = {}
        for name, wld in (("1024x4KiB", W.d2d_blocks(seed=0)),
                          ("65536x4KiB", W.d2d_blocks(seed=1, n=65536, pool_blocks=262144))):
            r2 = Resident(wld)
            s, km = timed(r2, [0], [sA], args.steps, args.warmup, 0)
            pl = K.kvcopy_plan(*r2.addrs[0], wld.batches[0].size)
            hbm_bytes = 2 * wld.batches[0].nbytes + pl.n_chunks * 24
            d2d[name] = {"GBps_payload": round(gbs(wld.batches[0].nbytes, s), 2),
                         "us_per_call": round(s * 1e6, 2), "kernel_us": round(km[0] * 1e3, 2),
                         "hbm_GBps_kernel": round(gbs(hbm_bytes, km[0] / 1e3), 1),
                         "frac_hbm_peak": round(gbs(hbm_bytes, km[0] / 1e3) / HBM_PEAK_GBS, 4)}
            img = r2.image(1)
            exp = np.full(wld.arenas[1].nbytes, wld.arenas[1].sentinel, np.uint8)
            b = wld.batches[0]
            sa, da = r2.addrs[0]
            oracle.copy(sa, da, b.size, [(r2.bases[0], wld.arenas[0].host_image())],
                        [(r2.bases[1], exp)])
            if not np.array_equal(img, exp):
                log(f"PARITY FAILURE in d2d {name}")
                sys.exit(3)
            log(f"  d2d {name}: {d2d[name]} (bit-exact)")
            r2.free()
        extras["d2d"] = d2d

    dom = 0 if kern_ms[0] >= kern_ms[1] else 1
    meas_ceil = extras.get("contiguous_memcpy_ceiling_GBps", {}).get(("h2d", "d2h")[dom])
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {
            "workload": "bidirectional KV block burst: 16,384 shuffled 4 KiB H2D + 16,384 shuffled "
                        "4 KiB D2H per step, concurrent on two streams, 65,536-block device pool, "
                        "mapped pinned host buffers",
            "descriptors_per_step": n_desc, "bytes_per_step": step_bytes,
            "max_wgs": max_wgs, "chunk_bytes": K.CHUNK_DEFAULT, "seed": 0,
        },
        "roofline": {
            "bound": "pcie",
            "kernel": KERNEL_NAMES[dom],
            "achieved": round(ach[dom], 3),
            "peak": PCIE_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(ach[dom] / PCIE_PEAK_GBS, 4),
            "traffic": measured_traffic(KERNEL_NAMES[dom]),
            "kernel_ms": round(kern_ms[dom], 4),
            "algorithmic_bytes_per_launch": algo[dom],
            "measured_ceiling": meas_ceil,
            "frac_of_measured_ceiling": round(ach[dom] / meas_ceil, 4) if meas_ceil else None,
            "other_kernel": {"dir": ("H2D", "D2H")[1 - dom], "achieved": round(ach[1 - dom], 3),
                             "kernel_ms": round(kern_ms[1 - dom], 4)},
        },
        "cpu_baseline": {
            "value": round(cpu_gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full steps (16,384 H2D + 16,384 D2H descriptors of 4 KiB each, "
                      f"per-descriptor memcpy between host images), {cpu_s:.1f} s",
        },
        "parity": "bit-exact vs oracle",
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
