"""Randomized GPU parity: 150 seeded batches of every shape the contract
allows (workloads.random_batch: any direction, 1-3,000 descriptors, sizes
8 B-256 KiB with zeros, coalescible runs, src and dst offsets independent
mod 16), each with a random copy loop / option flag, chunk size, workgroup
cap and stream, checked bit-exact against the oracle on the whole arenas.
The seed of a failing case is in the message."""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import _check, _say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_copy_amd import kvcopy
    return kvcopy


@pytest.mark.parametrize("block", range(5))
def test_random_batches(K, block):
    from block_copy_amd.harness import Resident
    flag_set = [0, 0, K.F_PIPELINE, K.F_PER_CHUNK, K.F_DYNAMIC, K.F_DESC_UPLOAD,
                K.F_NO_COALESCE, K.F_VALIDATE, K.F_DYNAMIC | K.F_DESC_UPLOAD, K.F_WG_PER_CHUNK,
                K.F_WG_PER_CHUNK | K.F_DESC_UPLOAD | K.F_DST_ORDER]
    streams = [None, torch.cuda.Stream()]
    for seed in range(block * 30, block * 30 + 30):
        rng = np.random.default_rng(10_000 + seed)
        wl = W.random_batch(seed)
        max_wgs = int(rng.choice([1, 2, 3, 7, 16, 64, 0, -1]))
        chunk = int(rng.choice([0, 16, 48, 4096, 16384, 1 << 20]))
        flags = int(rng.choice(flag_set))
        st = streams[int(rng.integers(0, 2))]
        res = Resident(wl)
        _say("random seed", seed, "n", wl.batches[0].n, "dir", wl.batches[0].dir, "max_wgs",
             max_wgs, "chunk", chunk, "flags", flags)
        res.submit(0, max_wgs, st, chunk_bytes=chunk, flags=flags)
        torch.cuda.synchronize()
        _check(res, [0], f"random seed {seed} max_wgs={max_wgs} chunk={chunk} flags={flags}")
        res.free()
