// order_kernel.hip -- destination order made on the GPU, for worklists that
// are uploaded to device memory (KVCOPY_F_DST_ORDER | KVCOPY_F_DESC_UPLOAD).
//
// Which chunks run together decides where a copy writes at any moment.  On
// MI355X, D2D gathers of random 4 KiB blocks with one workgroup per chunk
// ran about 10% faster when the worklist was grouped by 4 MiB destination
// region (the dispatcher starts workgroups in chunk order, so the
// workgroups in flight then write a narrow band of HBM).
// Grouping on the host by 4 MiB region is a counting sort of the records
// there (80-90 us for 65,536 records on the MI355X host), which leaves
// back-to-back calls host-bound.  Here the same grouping runs as two small kernels after the
// upload, on the same stream of the library's own, before the copy (the
// caller's stream waits for them); in a train of calls they run while the
// previous call's copy does:
//   1. kvcopy_order_count_kernel: each workgroup counts its records per
//      region key ((dst >> 22) & 255) in LDS and adds its counts into the
//      call's 256 global counters;
//   2. kvcopy_order_place_kernel: each workgroup turns the counters into the
//      first slot of every key (an exclusive scan in LDS), counts its own
//      records again, reserves a run of slots per key with one global atomic
//      add on the call's 256 cursors, and writes each record into a slot of
//      its run (slots handed out by LDS atomics).
// Both kernels visit the records in the same grid-stride order.  The
// counters and cursors sit in a 2 KiB header in front of the uploaded
// records; the host zeroes it in the staging ring and the upload carries the
// zeros, so nothing needs clearing on the device and calls on other streams
// (other ring regions) never share counters.  Within a key the records come
// in no set order: destinations do not overlap, so the bytes copied do not
// depend on it.
#include <hip/hip_runtime.h>

#include "kvcopy.h"
#include "kvcopy_internal.h"

namespace kvc {
namespace {

constexpr uint32_t kKeys = kOrderKeys;
static_assert(kKeys == kOrderThreads, "one key per thread of a workgroup");
// Records per thread per pass of the grid-stride loops: their loads are all
// issued before the first is used, so a workgroup's share (kOrderPerWG =
// kUnroll x kOrderThreads records) costs one memory latency, not four.
constexpr uint32_t kUnroll = kOrderPerWG / kOrderThreads;
static_assert(kUnroll * kOrderThreads == kOrderPerWG, "a workgroup's share is whole passes");

__device__ __forceinline__ uint32_t region_key(uint64_t dst)
{
    return (uint32_t)(dst >> kOrderShift) & (kKeys - 1);
}

// Adds this workgroup's records (records first, first + step, ... below n)
// into h[key]; kKeys marks a slot past the end.
__device__ __forceinline__ void count_keys(const ChunkRec *__restrict__ in, uint64_t n,
                                           uint64_t first, uint64_t step, uint32_t *h)
{
    for (uint64_t i0 = first; i0 < n; i0 += kUnroll * step) {
        uint32_t k[kUnroll];
#pragma unroll
        for (uint32_t u = 0; u < kUnroll; ++u) {
            // past the end: load the last record (no branch around the
            // loads, so all are in flight together) and drop its key
            const uint64_t i = i0 + u * step;
            const uint32_t key = region_key(in[i < n ? i : n - 1].dst);
            k[u] = i < n ? key : kKeys;
        }
#pragma unroll
        for (uint32_t u = 0; u < kUnroll; ++u)
            if (k[u] < kKeys)
                atomicAdd(&h[k[u]], 1u);
    }
}

__global__ __launch_bounds__(kOrderThreads) void kvcopy_order_count_kernel(
    const ChunkRec *__restrict__ in, uint32_t n, uint32_t *__restrict__ counts)
{
    __shared__ uint32_t h[kKeys];
    const uint32_t t = threadIdx.x;
    h[t] = 0;
    __syncthreads();
    const uint64_t step = (uint64_t)gridDim.x * kOrderThreads;
    count_keys(in, n, (uint64_t)blockIdx.x * kOrderThreads + t, step, h);
    __syncthreads();
    const uint32_t c = h[t];
    if (c != 0)
        atomicAdd(&counts[t], c);
}

__global__ __launch_bounds__(kOrderThreads) void kvcopy_order_place_kernel(
    const ChunkRec *__restrict__ in, uint32_t n, ChunkRec *__restrict__ out,
    const uint32_t *__restrict__ counts, uint32_t *__restrict__ cursors)
{
    __shared__ uint32_t first[kKeys];   // inclusive scan of counts
    __shared__ uint32_t h[kKeys];       // this workgroup's records per key, then its next slot
    const uint32_t t = threadIdx.x;
    const uint32_t mine = counts[t];
    first[t] = mine;
    h[t] = 0;
    __syncthreads();
    for (uint32_t s = 1; s < kKeys; s <<= 1) {
        const uint32_t v = t >= s ? first[t - s] : 0;
        __syncthreads();
        first[t] += v;
        __syncthreads();
    }
    const uint64_t step = (uint64_t)gridDim.x * kOrderThreads;
    const uint64_t begin = (uint64_t)blockIdx.x * kOrderThreads + t;
    count_keys(in, n, begin, step, h);
    __syncthreads();
    // thread t owns key t: its run of slots starts after the keys before it
    // and after the runs other workgroups reserved before this one
    const uint32_t c = h[t];
    h[t] = c != 0 ? first[t] - mine + atomicAdd(&cursors[t], c) : 0;
    __syncthreads();
    for (uint64_t i0 = begin; i0 < n; i0 += kUnroll * step) {
        ChunkRec r[kUnroll];
#pragma unroll
        for (uint32_t u = 0; u < kUnroll; ++u) {
            const uint64_t i = i0 + u * step;
            r[u] = in[i < n ? i : n - 1];
        }
#pragma unroll
        for (uint32_t u = 0; u < kUnroll; ++u) {
            if (i0 + u * step >= n)
                break;
            const uint32_t slot = atomicAdd(&h[region_key(r[u].dst)], 1u);
            if (slot < n)   // always: the runs of all workgroups tile [0, n)
                out[slot] = r[u];
        }
    }
}

}  // namespace

hipError_t launch_order(const ChunkRec *in, uint32_t n, ChunkRec *out, uint32_t *header,
                        hipStream_t stream, hipEvent_t start)
{
    if (n == 0)   // nothing to order (the kernels load record n - 1 past the end of a pass)
        return hipSuccess;
    uint64_t blocks = ((uint64_t)n + kOrderPerWG - 1) / kOrderPerWG;
    const uint32_t grid = (uint32_t)(blocks < kOrderMaxGrid ? (blocks ? blocks : 1) : kOrderMaxGrid);
    uint32_t *counts = header, *cursors = header + kOrderKeys;
    void *count_args[] = {(void *)&in, (void *)&n, (void *)&counts};
    hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(&kvcopy_order_count_kernel),
                                      dim3(grid), dim3(kOrderThreads), count_args, 0, stream,
                                      start, nullptr, 0);
    if (e != hipSuccess)
        return e;
    void *place_args[] = {(void *)&in, (void *)&n, (void *)&out, (void *)&counts,
                          (void *)&cursors};
    return hipExtLaunchKernel(reinterpret_cast<const void *>(&kvcopy_order_place_kernel),
                              dim3(grid), dim3(kOrderThreads), place_args, 0, stream, nullptr,
                              nullptr, 0);
}

}  // namespace kvc
