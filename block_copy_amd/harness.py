"""Arena plumbing for the tests, the smoke check and bench.py.

Allocates the arenas of a ``workloads.Workload`` (device memory through
torch, mapped pinned host memory through the library's allocator), fills
them as the workload says, turns (arena, offset) descriptors into absolute
addresses and submits batches through the C ABI.  It computes nothing of
the copy itself.
"""
from __future__ import annotations

import numpy as np
import torch

from . import kvcopy as K


class Resident:
    """A workload's arenas, resident on the GPU or in mapped pinned host memory."""

    def __init__(self, wl, device: str = "cuda:0"):
        self.wl = wl
        self.device = torch.device(device)
        self.bufs = []
        self.bases = []
        for a in wl.arenas:
            if a.where == "device":
                t = torch.empty(a.nbytes, dtype=torch.uint8, device=self.device)
                self.bufs.append(t)
                self.bases.append(t.data_ptr())
            elif a.where == "host":
                hb = K.HostBuffer(a.nbytes)
                self.bufs.append(hb)
                self.bases.append(hb.ptr)
            else:
                raise ValueError(a.where)
        self.fill()
        self.addrs = [b.addresses(self.bases) for b in wl.batches]

    def fill(self, sentinel: int | None = None):
        """(Re)fill every arena; ``sentinel`` overrides sentinel arenas' byte."""
        for a, buf in zip(self.wl.arenas, self.bufs):
            val = a.sentinel if sentinel is None else sentinel
            if a.where == "device":
                if a.fill == "sentinel":
                    buf.fill_(val)
                else:
                    buf.copy_(torch.from_numpy(a.host_image()))
            else:
                if a.fill == "sentinel":
                    buf.array.fill(val)
                else:
                    buf.array[:] = a.host_image()
        torch.cuda.synchronize(self.device)

    def image(self, i: int) -> np.ndarray:
        """Host copy of arena i's current bytes."""
        buf = self.bufs[i]
        if isinstance(buf, torch.Tensor):
            return buf.cpu().numpy()
        return buf.array.copy()

    def submit(self, batch_idx: int, max_wgs: int = K.WGS_ALL, stream=None, **kw) -> int:
        b = self.wl.batches[batch_idx]
        s, d = self.addrs[batch_idx]
        st = getattr(stream, "cuda_stream", stream)
        return K.kvcopy_batch(s, d, b.size, b.dir, max_wgs, st, **kw)

    def free(self):
        for buf in self.bufs:
            if isinstance(buf, K.HostBuffer):
                buf.free()
        self.bufs = []
