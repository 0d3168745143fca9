// hbm_probe.hip -- measurement only: what HBM delivers for a list of scattered
// blocks when they are only read, or only written.  Not part of the copy path.
//
// A D2D gather/scatter of random 4 KiB blocks reads every block once and
// writes every block once.  HBM reads and writes share each channel's data
// bus, so the copy cannot take less time than reading the same source blocks
// plus writing the same destination blocks, each at the rate HBM sustains
// for that scattered pattern.  These two kernels time the two halves with
// the copy kernel's own access shapes (one wavefront per block, 1 KiB per
// wavefront instruction, 16-byte buffer accesses, plain loads, nontemporal
// stores), so bench.py can report the copy against that composite ceiling
// beside the published 8 TB/s.
//
// Both take a device array of n block addresses (8-byte aligned, each block
// `block_bytes` long, a multiple of 16 of at most 16 KiB) and optional
// events that the launch records at the kernel's own start and end.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kWaves = 4;
constexpr uint32_t kRow = 1024;        // one wavefront instruction: 64 lanes x 16 B
constexpr uint32_t kMaxBlock = 16384;
constexpr int kRsrcWord3 = 0x00020000; // raw buffer, 32-bit format, no swizzle or stride

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(uint64_t base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), 0, (int)bytes,
                                             kRsrcWord3);
}

// Reads every block and folds the words into one value per lane; the value
// is stored to `sink` only if it equals `never`, which keeps the loads live.
__global__ __launch_bounds__(64 * kWaves) void gather_read_kernel(const uint64_t *__restrict__ addrs,
                                                                 uint32_t n, uint32_t block_bytes,
                                                                 uint32_t never,
                                                                 uint32_t *__restrict__ sink)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b >= n)
        return;
    const __amdgpu_buffer_rsrc_t r = rsrc(addrs[b], block_bytes);
    v4u v[kMaxBlock / kRow];
#pragma unroll
    for (uint32_t j = 0; j < kMaxBlock / kRow; ++j)
        if (j * kRow < block_bytes)
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(lane * 16u + j * kRow), 0, 0);
    uint32_t acc = 0;
#pragma unroll
    for (uint32_t j = 0; j < kMaxBlock / kRow; ++j)
        if (j * kRow < block_bytes)
            acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if (acc == never)
        sink[lane] = acc;
}

// Writes a pattern over every block (nontemporal stores, as the copy does).
__global__ __launch_bounds__(64 * kWaves) void scatter_write_kernel(const uint64_t *__restrict__ addrs,
                                                                   uint32_t n, uint32_t block_bytes,
                                                                   uint32_t pattern)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b >= n)
        return;
    const __amdgpu_buffer_rsrc_t r = rsrc(addrs[b], block_bytes);
    const v4u v = {pattern, pattern, pattern, pattern};
#pragma unroll
    for (uint32_t j = 0; j < kMaxBlock / kRow; ++j)
        if (j * kRow < block_bytes)
            __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)(lane * 16u + j * kRow), 0, 2);
}

bool bad_args(const uint64_t *addrs, uint32_t n, uint32_t block_bytes)
{
    return !addrs || n == 0 || n > (1u << 30) || block_bytes == 0 || (block_bytes & 15u) ||
           block_bytes > kMaxBlock;
}

}  // namespace

extern "C" {

// Read n scattered blocks (device array `addrs` of block addresses) on
// `stream`.  `sink` is a device buffer of at least 64 uint32 that is written
// only if the folded data equals `never`.  `start` and `stop` (either may be
// null) are recorded at the kernel's own start and end.  Returns a
// hipError_t value; hipErrorInvalidValue for a null pointer, n == 0 or above 2^30, or a
// block size that is not a multiple of 16 in (0, 16 KiB].
int kvload_gather_read(const uint64_t *addrs, uint32_t n, uint32_t block_bytes, uint32_t never,
                       uint32_t *sink, hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    if (bad_args(addrs, n, block_bytes) || !sink)
        return (int)hipErrorInvalidValue;
    void *args[] = {(void *)&addrs, (void *)&n, (void *)&block_bytes, (void *)&never, (void *)&sink};
    return (int)hipExtLaunchKernel(reinterpret_cast<const void *>(&gather_read_kernel),
                                   dim3((n + kWaves - 1) / kWaves), dim3(64 * kWaves), args, 0,
                                   stream, start, stop, 0);
}

// Fill n scattered blocks with the 32-bit `pattern` on `stream`; same
// argument rules and events as kvload_gather_read.
int kvload_scatter_write(const uint64_t *addrs, uint32_t n, uint32_t block_bytes, uint32_t pattern,
                         hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    if (bad_args(addrs, n, block_bytes))
        return (int)hipErrorInvalidValue;
    void *args[] = {(void *)&addrs, (void *)&n, (void *)&block_bytes, (void *)&pattern};
    return (int)hipExtLaunchKernel(reinterpret_cast<const void *>(&scatter_write_kernel),
                                   dim3((n + kWaves - 1) / kWaves), dim3(64 * kWaves), args, 0,
                                   stream, start, stop, 0);
}

}  // extern "C"
