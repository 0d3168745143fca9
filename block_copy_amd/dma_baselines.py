"""DMA baselines measured in a process of their own, without torch.

torch ships its own HIP runtime, and in a process that has imported torch
every HIP call (libkvcopy.so's included) goes to that copy.  The runtime
bundled with this torch build does not export hipMemcpyBatchAsync, the
runtime's batched DMA path (the counterpart of the batched DMA API that the
vLLM PR #42212 report, section "implementation breakdown", measures as the
baseline at 6-7 GB/s).  This module therefore runs in a fresh interpreter
that loads ROCm's own runtime, allocates the arenas of the benchmark
workloads with plain hipMalloc / hipHostMalloc, and times, per workload:
  - one hipMemcpyAsync per (coalesced) range on one stream;
  - one hipMemcpyBatchAsync call for the whole list, when exported.
It computes nothing of the copy itself and checks only return codes (this
is a timing baseline; the kernel's bytes are checked elsewhere).

    python -m block_copy_amd.dma_baselines     # prints one JSON object
"""
from __future__ import annotations

import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _workloads(W):
    return [("kv_h2d_16384x4KiB", W.kv_blocks(seed=0, directions="h2d")),
            ("kv_d2h_16384x4KiB", W.kv_blocks(seed=0, directions="d2h")),
            ("d2d_1024x4KiB", W.d2d_blocks(seed=0)),
            ("h2d_mixed_16", W.h2d_mixed(seed=0, n=16)),
            ("h2d_mixed_256", W.h2d_mixed(seed=0, n=256)),
            ("h2d_mixed_4096", W.h2d_mixed(seed=0, n=4096))]


def main() -> int:
    if "torch" in sys.modules:
        raise RuntimeError("dma_baselines must run in a process without torch")
    import numpy as np

    import workloads as W
    from block_copy_amd import hiprt
    from block_copy_amd import kvcopy as K

    kinds = {(True, False): hiprt.H2D_KIND, (False, True): hiprt.D2H_KIND,
             (False, False): hiprt.D2D_KIND}
    st = hiprt.stream_create()
    out = {"hip_runtime_version": hiprt.runtime_version(),
           "hipMemcpyBatchAsync_exported": hiprt.has_memcpy_batch(), "rows": {}}
    for name, wl in _workloads(W):
        bases, frees = [], []
        for a in wl.arenas:
            if a.where == "device":
                p = hiprt.device_alloc(a.nbytes)
                hiprt.memset(p, 0, a.nbytes)
                frees.append((hiprt.device_free, p))
            else:
                p = hiprt.host_alloc_mapped(a.nbytes)
                frees.append((hiprt.host_free, p))
            bases.append(p)
        b = wl.batches[0]
        s, d = b.addresses(bases)
        cs, cd, cz = K.kvcopy_coalesce(s, d, b.size)
        src_host = wl.arenas[int(b.src_arena[0])].where == "host"
        dst_host = wl.arenas[int(b.dst_arena[0])].where == "host"
        kind = kinds[(src_host, dst_host)]
        row = {"descriptors": int(b.n), "ranges": int(len(cz)), "bytes": int(b.nbytes)}
        reps = 3
        hiprt.stream_sync(st)
        t0 = time.perf_counter()
        for _ in range(reps):
            for s_, d_, z_ in zip(cs.tolist(), cd.tolist(), cz.tolist()):
                hiprt.memcpy_async(d_, s_, z_, kind, st)
        hiprt.stream_sync(st)
        dt = (time.perf_counter() - t0) / reps
        row["per_fragment"] = {"GBps": round(b.nbytes / dt / 1e9, 3), "ms_per_call": round(dt * 1e3, 3)}
        if hiprt.has_memcpy_batch():
            # With copy attributes first (location hints, stream order), then
            # without: the runtime's header marks the attributes unsupported.
            errors = {}
            for attrs in (True, False):
                rc = hiprt.memcpy_batch_async(cd, cs, cz, st, src_host, dst_host, attrs)
                hiprt.stream_sync(st)
                if rc != 0:
                    errors["with_attrs" if attrs else "no_attrs"] = rc
                    continue
                t0 = time.perf_counter()
                for _ in range(reps):
                    hiprt.check(hiprt.memcpy_batch_async(cd, cs, cz, st, src_host, dst_host, attrs),
                                "hipMemcpyBatchAsync")
                hiprt.stream_sync(st)
                dt = (time.perf_counter() - t0) / reps
                row["hipMemcpyBatchAsync"] = {"GBps": round(b.nbytes / dt / 1e9, 3),
                                              "ms_per_call": round(dt * 1e3, 3), "attrs": attrs}
                break
            if errors:
                row["hipMemcpyBatchAsync_errors"] = errors
        out["rows"][name] = row
        print(f"{name}: {row}", file=sys.stderr, flush=True)
        for f, p in frees:
            f(p)
    hiprt.check(hiprt.hip.hipStreamDestroy(st), "hipStreamDestroy")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
