"""Expected arena images from the oracle, and comparison helpers for GPU tests."""
from __future__ import annotations

import numpy as np

import oracle


def initial_images(wl, sentinel=None, only=None):
    """Initial bytes of each arena (None for arenas not in `only`)."""
    out = []
    for i, a in enumerate(wl.arenas):
        if only is not None and i not in only:
            out.append(None)
        elif a.fill == "sentinel":
            out.append(np.full(a.nbytes, a.sentinel if sentinel is None else sentinel, np.uint8))
        else:
            out.append(a.host_image().copy())
    return out


def expected_images(wl, batch_ids, bases, sentinel=None):
    """Apply the given batches (in order) with the oracle to fresh images.

    The images are keyed by arena index; only arenas that some batch reads or
    writes are built.  Source bytes are taken from a snapshot made before
    each batch, as the copy reads sources that it does not write.
    """
    touched = set()
    for k in batch_ids:
        b = wl.batches[k]
        touched |= set(b.src_arena.tolist()) | set(b.dst_arena.tolist())
    imgs = initial_images(wl, sentinel, only=touched)
    for k in batch_ids:
        b = wl.batches[k]
        s, d = b.addresses(bases)
        src_ids = sorted(set(b.src_arena.tolist()))
        dst_ids = sorted(set(b.dst_arena.tolist()))
        snap = {i: (imgs[i].copy() if i in dst_ids else imgs[i]) for i in src_ids}
        oracle.copy(s, d, b.size, [(bases[i], snap[i]) for i in src_ids],
                    [(bases[i], imgs[i]) for i in dst_ids])
    return imgs


def assert_same(actual: np.ndarray, expected: np.ndarray, what: str, wl=None, batch=None,
                bases=None, arena=None):
    """Bit-exact comparison; on failure name the first differing byte and its descriptor."""
    if actual.shape == expected.shape and np.array_equal(actual, expected):
        return
    if actual.shape != expected.shape:
        raise AssertionError(f"{what}: shape {actual.shape} != {expected.shape}")
    bad = np.flatnonzero(actual != expected)
    first = int(bad[0])
    msg = (f"{what}: {bad.size} bytes differ; first at offset {first}: "
           f"got {actual[first]:#04x}, expected {expected[first]:#04x}")
    if wl is not None and batch is not None and arena is not None:
        b = wl.batches[batch]
        hit = np.flatnonzero((b.dst_arena == arena) & (b.dst_off <= first) &
                             (b.dst_off + b.size > first))
        if hit.size:
            i = int(hit[0])
            msg += (f"; inside descriptor {i} (dst_off {int(b.dst_off[i])}, size {int(b.size[i])},"
                    f" src_off {int(b.src_off[i])}, src_arena {int(b.src_arena[i])})")
        else:
            msg += "; outside every destination range (guard bytes changed)"
    raise AssertionError(msg)
