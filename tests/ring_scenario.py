"""Staging-ring safety scenario (run by test_gpu_parity.py in a fresh process).

300 D2D calls with different worklists go on one stream. Each runs on a
single workgroup (2,048 chunks of 64 bytes per wavefront; every other call
forces the per-chunk loop), so the GPU falls far behind the host. The 16 MiB
staging ring (192 KiB of worklist per call) therefore fills several times,
and the host must wait for ring space. Every call writes its own destination
blocks, so a region recycled before its kernel finished would make some call
copy another call's descriptors, and that call's destinations would keep the
sentinel. Exit status 0 means every byte matches the oracle and the host did
wait.
"""
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)


def main() -> int:
    import numpy as np
    import torch

    import workloads as W
    from block_copy_amd import kvcopy as K
    from block_copy_amd.harness import Resident
    from expect import expected_images

    wl = W.distinct_calls(seed=12)
    res = Resident(wl)
    st = torch.cuda.Stream()
    t0 = time.perf_counter()
    for i in range(len(wl.batches)):
        res.submit(i, 1, st, flags=K.F_PER_CHUNK if i % 2 else 0)
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    print(f"submitted in {t1 - t0:.3f} s, all done after {t2 - t0:.3f} s", flush=True)
    exp = expected_images(wl, list(range(len(wl.batches))), res.bases)
    got = res.image(1)
    if not np.array_equal(got, exp[1]):
        bad = int(np.flatnonzero(got != exp[1])[0])
        print(f"MISMATCH at destination offset {bad}", flush=True)
        return 1
    # The host had to wait for ring space: most of the GPU time passed
    # inside the submission loop.
    if not t1 - t0 > 0.5 * (t2 - t0):
        print("the ring never filled: the scenario did not test what it should", flush=True)
        return 2
    res.free()
    print("ok", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
