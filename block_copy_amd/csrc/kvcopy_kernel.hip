// kvcopy_kernel.hip -- the persistent, workgroup-capped copy kernel (gfx950).
//
// Work unit: one chunk of the worklist (at most chunk_bytes, never crossing a
// range; FreeToken issue #751 "gather missed experts with a few TMA
// bulk-copy CTAs", section "What we changed", which deals such chunks to a
// few CTAs).  The grid is persistent, as in the vLLM PR #42212 report
// ("Triton fast path for small CPU->GPU swap_blocks_batch"), section "key
// source snippet", where a few programs loop over all jobs; here the job is a
// byte-bounded chunk instead of a whole descriptor, so a 1 MiB row is shared
// by many wavefronts while small rows are not left waiting.  The grid is
// capped by max_wgs (PegaFlow issue #408, "Follow-up", item 1: a bounded
// grid).  Each wavefront takes an equal contiguous share of the chunk list.
//
// Data path (CDNA4): each lane moves 16-byte vectors with
// buffer_load_dwordx4 / nontemporal buffer_store_dwordx4, lanes interleaved
// so that one wavefront instruction covers 1 KiB of contiguous bytes.  A wavefront
// issues the loads for up to 16 KiB (16 vectors per lane, 64 VGPRs) before
// the first store, so a single wavefront keeps up to 16 KiB of reads in
// flight; the worklist records are fetched 64 at a time and one batch
// ahead.  Addresses only need 8-byte alignment: gfx950 serves
// 8-byte-aligned dwordx4 accesses directly, so no head peeling or register
// shifting is needed when src and dst differ mod 16.  A range whose size is
// an odd multiple of 8 ends in one 8-byte word, moved by lane 0.
#include <hip/hip_runtime.h>

#include "kvcopy.h"
#include "kvcopy_internal.h"

namespace kvc {
namespace {

#include "copy_chunk.h"

// The persistent loop.  Wavefront w of W owns the contiguous chunk range
// [w*C/W, (w+1)*C/W): every wavefront gets the same number of chunks to
// within one, and every chunk is at most chunk_bytes, so the bytes are
// balanced.  The wavefront fetches its worklist records 64 at a time, one
// record per lane, with vector loads (the worklist may sit in pinned host
// memory: one round trip per 64 chunks), prefetching the next 64 while it
// copies the current ones, and hands each record to the whole wavefront with
// v_readlane.
struct Rec {
    uint64_t src, dst;
    uint32_t bytes;
};

__device__ __forceinline__ Rec load_rec(const ChunkRec *recs, uint32_t idx, bool valid)
{
    Rec r{0, 0, 0};
    if (valid) {
        const KVC_GLOBAL uint64_t *p =
            (const KVC_GLOBAL uint64_t *)reinterpret_cast<uintptr_t>(recs + idx);
        r.src = p[0];
        r.dst = p[1];
        r.bytes = (uint32_t)p[2];
    }
    return r;
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, uint32_t j)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, j);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), j);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void copy_worklist(const ChunkRec *__restrict__ recs, uint32_t n_chunks)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t nw = gridDim.x * kWavesPerWG;
    const uint32_t w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWG + (threadIdx.x >> 6));
    const uint32_t lo = (uint32_t)((uint64_t)w * n_chunks / nw);
    const uint32_t hi = (uint32_t)((uint64_t)(w + 1) * n_chunks / nw);
    if (lo >= hi)
        return;
    Rec cur = load_rec(recs, lo + lane, lo + lane < hi);
    for (uint32_t base = lo; base < hi; base += 64u) {
        const uint32_t cnt = hi - base < 64u ? hi - base : 64u;
        const uint32_t nb = base + 64u;
        const Rec nxt = load_rec(recs, nb + lane, nb < hi && nb + lane < hi);   // prefetch
        for (uint32_t j = 0; j < cnt; ++j)
            copy_chunk(lane_u64(cur.src, j), lane_u64(cur.dst, j),
                       __builtin_amdgcn_readlane(cur.bytes, j), lane);
        cur = nxt;
    }
}

// One symbol per direction, so that profiles and counters separate them.
__global__ __launch_bounds__(kThreadsPerWG) void kvcopy_h2d_kernel(const ChunkRec *__restrict__ recs,
                                                                   uint32_t n_chunks)
{
    copy_worklist(recs, n_chunks);
}

__global__ __launch_bounds__(kThreadsPerWG) void kvcopy_d2h_kernel(const ChunkRec *__restrict__ recs,
                                                                   uint32_t n_chunks)
{
    copy_worklist(recs, n_chunks);
}

__global__ __launch_bounds__(kThreadsPerWG) void kvcopy_d2d_kernel(const ChunkRec *__restrict__ recs,
                                                                   uint32_t n_chunks)
{
    copy_worklist(recs, n_chunks);
}

}  // namespace

hipError_t launch_copy(const ChunkRec *recs, uint32_t n_chunks, uint32_t grid, int dir,
                       hipStream_t stream)
{
    const void *fn = dir == KVCOPY_H2D   ? reinterpret_cast<const void *>(&kvcopy_h2d_kernel)
                     : dir == KVCOPY_D2H ? reinterpret_cast<const void *>(&kvcopy_d2h_kernel)
                                         : reinterpret_cast<const void *>(&kvcopy_d2d_kernel);
    void *args[] = {(void *)&recs, (void *)&n_chunks};
    return hipLaunchKernel(fn, dim3(grid), dim3(kThreadsPerWG), args, 0, stream);
}

}  // namespace kvc
