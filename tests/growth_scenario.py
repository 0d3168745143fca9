"""Ring growth with uploaded, GPU-ordered worklists in flight (run by
test_gpu_parity.py in a fresh process, where the staging ring still has its
initial 16 MiB).

Calls with KVCOPY_F_DESC_UPLOAD | KVCOPY_F_DST_ORDER (the worklist copied to
the ring's device twin and grouped there by two order kernels on the
library's upload stream) are queued on one stream, some on a single
workgroup so that the GPU falls behind. Then a call whose worklist needs more
than a quarter of the ring (200,000 records, 4.6 MiB) makes the library grow
the ring: it must wait for the queued kernels and for the upload stream
before it frees the old host ring and device twin. More calls follow on the
new ring. Exit status 0 means every destination byte matches the oracle.
"""
import os
import sys

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

    small = W.d2d_blocks(seed=61, n=16384, pool_blocks=65536)
    big = W.d2d_blocks(seed=62, n=200_000, pool_blocks=262144, block=64)
    rs, rb = Resident(small), Resident(big)
    st = torch.cuda.Stream()
    fl = K.F_DESC_UPLOAD | K.F_DST_ORDER
    for i in range(12):
        rs.submit(0, 1 if i % 4 == 0 else 0, st, flags=fl | (K.F_WG_PER_CHUNK if i % 2 else 0))
    rb.submit(0, 0, st, flags=fl | K.F_WG_PER_CHUNK)     # grows the ring
    for i in range(6):
        rs.submit(0, 0, st, flags=fl | (K.F_WG_PER_CHUNK if i % 2 else 0))
    torch.cuda.synchronize()
    for name, r, wl in (("small", rs, small), ("big", rb, big)):
        exp = expected_images(wl, [0], r.bases)
        got = r.image(1)
        if not np.array_equal(got, exp[1]):
            bad = int(np.flatnonzero(got != exp[1])[0])
            print(f"MISMATCH in the {name} batch at destination offset {bad}", flush=True)
            return 1
    rs.free()
    rb.free()
    print("ok", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
