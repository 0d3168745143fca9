// device_batch.hip -- a batch whose descriptor list and count live in device
// memory: fixed launch shapes, no host planning, capturable in a HIP graph.
//
// FreeToken issue #751 ("gather missed experts with a few TMA bulk-copy
// CTAs"), section "What we changed": the gather reads the miss count on the
// device, so the launch has a fixed shape and a graph can capture it.  Here
// two kernels run on the caller's stream:
//   1. kvcopy_device_plan_kernel (one workgroup): reads n from device memory,
//      checks 8-byte alignment, and writes the exclusive prefix sum of the
//      per-descriptor chunk counts, ceil(size / chunk), into the workspace
//      (the same chunk numbering as the host planner, without coalescing);
//   2. kvcopy_device_copy_kernel (max_wgs workgroups): wavefront w of W
//      copies chunks [w*C/W, (w+1)*C/W), finding its first descriptor by a
//      binary search over the prefix and walking forward from there.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "kvcopy.h"
#include "kvcopy_internal.h"

namespace kvc {
namespace {

#include "copy_chunk.h"

constexpr int kPlanThreads = 1024;

struct DevWorkspace {
    uint64_t status;   // 0 ok, KVCOPY_DEVICE_BAD_ALIGN, KVCOPY_DEVICE_TOO_MANY_CHUNKS
    uint64_t n;        // descriptors planned (the device count, clamped to max_n)
    uint64_t total;    // chunks (0 when status != 0)
    uint64_t reserved;
    uint64_t begin[1]; // n + 1 entries: exclusive prefix of chunk counts
};

__device__ __forceinline__ uint64_t wave_incl_scan(uint64_t v, uint32_t lane)
{
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint64_t o = __shfl_up(v, d, 64);
        if (lane >= d)
            v += o;
    }
    return v;
}

__global__ __launch_bounds__(kPlanThreads) void kvcopy_device_plan_kernel(
    const uint64_t *__restrict__ src, const uint64_t *__restrict__ dst,
    const uint64_t *__restrict__ size, const uint64_t *__restrict__ d_n, uint64_t max_n,
    uint32_t chunk, DevWorkspace *__restrict__ ws, uint64_t *__restrict__ status_out)
{
    __shared__ uint64_t wave_tot[kPlanThreads / 64];
    __shared__ uint64_t carry_s;
    __shared__ uint32_t bad_s;
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint64_t n_dev = *d_n;
    const uint64_t n = n_dev < max_n ? n_dev : max_n;
    if (tid == 0) {
        carry_s = 0;
        bad_s = 0;
    }
    __syncthreads();
    uint32_t bad = 0;
    for (uint64_t tile = 0; tile < n; tile += kPlanThreads) {
        const uint64_t i = tile + tid;
        uint64_t c = 0;
        if (i < n) {
            const uint64_t z = size[i];
            bad |= (uint32_t)((src[i] | dst[i] | z) & 7u);
            c = z / chunk + (z % chunk != 0);
        }
        const uint64_t incl = wave_incl_scan(c, lane);
        if (lane == 63)
            wave_tot[wave] = incl;
        __syncthreads();
        uint64_t before = carry_s;
        for (uint32_t w = 0; w < wave; ++w)
            before += wave_tot[w];
        if (i < n)
            ws->begin[i] = before + incl - c;
        __syncthreads();
        if (tid == kPlanThreads - 1)
            carry_s = before + incl;   // the last thread holds the tile's running total
        __syncthreads();
    }
    if (bad)
        atomicOr(&bad_s, 1u);
    __syncthreads();
    if (tid == 0) {
        const uint64_t total = carry_s;
        ws->begin[n] = total;
        ws->n = n;
        uint64_t status = bad_s ? (uint64_t)KVCOPY_DEVICE_BAD_ALIGN : 0;
        if (!status && total >= ((uint64_t)1 << 31))
            status = KVCOPY_DEVICE_TOO_MANY_CHUNKS;
        ws->status = status;
        ws->total = status ? 0 : total;
        if (status_out)
            *status_out = status;
    }
}

// Last index i in [0, n] with begin[i] <= k (begin is non-decreasing and begin[0] == 0).
__device__ __forceinline__ uint64_t find_desc(const uint64_t *begin, uint64_t n, uint64_t k)
{
    uint64_t lo = 0, hi = n;   // invariant: begin[lo] <= k < begin[hi + 1] ... searched in [lo, hi]
    while (lo < hi) {
        const uint64_t mid = (lo + hi + 1) >> 1;
        if (begin[mid] <= k)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kThreadsPerWG) void kvcopy_device_copy_kernel(
    const uint64_t *__restrict__ src, const uint64_t *__restrict__ dst,
    const uint64_t *__restrict__ size, uint32_t chunk, const DevWorkspace *__restrict__ ws)
{
    if (ws->status != 0)
        return;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t nw = gridDim.x * kWavesPerWG;
    const uint32_t w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWG + (threadIdx.x >> 6));
    const uint64_t total = ws->total, n = ws->n;
    const uint64_t lo = total * w / nw, hi = total * (w + 1) / nw;
    if (lo >= hi)
        return;
    const uint64_t *begin = ws->begin;
    uint64_t i = find_desc(begin, n, lo);
    for (uint64_t k = lo; k < hi; ++k) {
        while (begin[i + 1] <= k)      // skip to the descriptor that owns chunk k
            ++i;
        const uint64_t off = (k - begin[i]) * chunk;
        const uint64_t left = size[i] - off;
        copy_chunk(src[i] + off, dst[i] + off, (uint32_t)(left < chunk ? left : chunk), lane);
    }
}

}  // namespace

uint64_t device_workspace_bytes(uint64_t max_n)
{
    return (offsetof(DevWorkspace, begin) + 8 * (max_n + 1) + 255) / 256 * 256;
}

hipError_t launch_device_batch(const uint64_t *src, const uint64_t *dst, const uint64_t *size,
                               const uint64_t *d_n, uint64_t max_n, uint32_t chunk, uint32_t grid,
                               void *workspace, uint64_t *status_out, hipStream_t stream)
{
    DevWorkspace *ws = reinterpret_cast<DevWorkspace *>(workspace);
    {
        void *args[] = {(void *)&src, (void *)&dst, (void *)&size, (void *)&d_n, (void *)&max_n,
                        (void *)&chunk, (void *)&ws, (void *)&status_out};
        const hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void *>(&kvcopy_device_plan_kernel), dim3(1),
                            dim3(kPlanThreads), args, 0, stream);
        if (e != hipSuccess)
            return e;
    }
    const DevWorkspace *cws = ws;
    void *args[] = {(void *)&src, (void *)&dst, (void *)&size, (void *)&chunk, (void *)&cws};
    return hipLaunchKernel(reinterpret_cast<const void *>(&kvcopy_device_copy_kernel), dim3(grid),
                           dim3(kThreadsPerWG), args, 0, stream);
}

// ---- the library's own workspace (kvcopy_batch_device_noalloc) -------------
//
// A workspace for KVCOPY_NOALLOC_MAX_N descriptors in a file-scope device
// array, so that a call needs no allocation at all.  Each GPU the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address comes
// from hipGetSymbolAddress, once per device (with that device current), and
// only that address is ever handed to a kernel.  Every call on a device uses
// the same array; the plan kernel rewrites every word the copy kernel reads,
// so nothing in it needs clearing between calls.
constexpr uint64_t kNoallocBytes = (32 + 8 * (KVCOPY_NOALLOC_MAX_N + 1) + 255) / 256 * 256;
static_assert(offsetof(DevWorkspace, begin) == 32, "workspace header layout");
static __device__ __align__(256) uint8_t scratch[kNoallocBytes];

namespace {

std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;   // device ordinal -> device address of `scratch`

}  // namespace

uint64_t noalloc_workspace_bytes()
{
    return kNoallocBytes;
}

hipError_t noalloc_workspace(int device, void **out)
{
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if ((size_t)device < g_scratch_ptr.size() && g_scratch_ptr[device] != nullptr) {
        *out = g_scratch_ptr[device];
        return hipSuccess;
    }
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return e;
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u))
        return hipErrorInvalidSymbol;
    if ((size_t)device >= g_scratch_ptr.size())
        g_scratch_ptr.resize((size_t)device + 1, nullptr);
    g_scratch_ptr[device] = ptr;
    *out = ptr;
    return hipSuccess;
}

}  // namespace kvc
