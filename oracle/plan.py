"""Oracle for the host-side planning steps: coalescing and chunking.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and bench.py's
cpu_baseline leg, never by the product library.  Plain Python loops, written
from the definitions below; no blocking, vectorisation or reordering.

Coalescing -- PegaFlow issue #408 ("Kernel transfer backend causes decode TPOT
tail spikes under concurrent KV transfers"), section "Relevant
implementation": the memcpy backend merges adjacent ranges before it submits
one copy per merged range.  The page gives no rule beyond that.  Reading
taken: walk the list once in order; drop zero-size descriptors; a descriptor
joins the range built so far when its source starts where that range's source
ends AND its destination starts where that range's destination ends.  No
sort.  Merging never changes what is copied where.

Chunking -- FreeToken issue #751 ("gather missed experts with a few TMA
bulk-copy CTAs"), section "What we changed": the call's rows are cut into
chunks of at most 16 KiB, each inside one row.  Reading taken: range i of
size s_i is cut into c_i = ceil(s_i / CHUNK) chunks; chunk j of range i covers
bytes [j*CHUNK, min((j+1)*CHUNK, s_i)); chunks are numbered range after range,
so range i owns chunk numbers [P_i, P_i + c_i) with P the exclusive prefix sum
of the c_i.
"""
from __future__ import annotations

CHUNK_DEFAULT = 16384


def coalesce(src, dst, size):
    """Merge list-consecutive descriptors adjacent in both src and dst.

    Returns three lists (src, dst, size) of the merged ranges.
    """
    out_src, out_dst, out_size = [], [], []
    for s, d, n in zip(src, dst, size):
        s, d, n = int(s), int(d), int(n)
        if n == 0:
            continue
        if out_size and out_src[-1] + out_size[-1] == s and out_dst[-1] + out_size[-1] == d:
            out_size[-1] += n
        else:
            out_src.append(s)
            out_dst.append(d)
            out_size.append(n)
    return out_src, out_dst, out_size


def chunk_counts(size, chunk_bytes=CHUNK_DEFAULT):
    """c_i = ceil(size_i / chunk_bytes) for every range."""
    return [(int(n) + chunk_bytes - 1) // chunk_bytes for n in size]


def chunk_begin(size, chunk_bytes=CHUNK_DEFAULT):
    """Exclusive prefix sum of the chunk counts; one more entry than ranges."""
    begin = [0]
    for c in chunk_counts(size, chunk_bytes):
        begin.append(begin[-1] + c)
    return begin


def chunks(src, dst, size, chunk_bytes=CHUNK_DEFAULT):
    """The chunk worklist: (src_addr, dst_addr, bytes) for every chunk, in chunk-number order."""
    out = []
    for s, d, n in zip(src, dst, size):
        s, d, n = int(s), int(d), int(n)
        j = 0
        while j * chunk_bytes < n:
            lo = j * chunk_bytes
            hi = min(lo + chunk_bytes, n)
            out.append((s + lo, d + lo, hi - lo))
            j += 1
    return out
