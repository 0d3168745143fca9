// gemv_load.hip -- a synthetic batch-1 decode loop used only to measure how a
// copy batch disturbs co-running decode.  Not part of the copy path.
//
// PegaFlow issue #408 ("Kernel transfer backend causes decode TPOT tail
// spikes under concurrent KV transfers"), sections "Test setup" and
// "Results": decode inter-token latency (p50/p99/max) is measured while
// bursts of KV transfers run on other streams.  The model decode is replaced
// here by a chain of bf16 matrix-vector products with distinct weights, which
// streams HBM the way batch-1 decode does.
//
// y[r] = sum_k W[r, k] * x[k], W row-major [rows, cols] bf16, x and y bf16,
// fp32 accumulation.  One wavefront per output row: lanes read 16-byte
// pieces (8 bf16) of the row, 1 KiB per wavefront instruction, multiply with
// the matching piece of x (read through the caches; every row re-reads the
// same x), and reduce across the wavefront.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kWaves = 4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0;                                   // NaN
    u += 0x7fffu + ((u >> 16) & 1u);                     // round to nearest even
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float dot8(v4u w, v4u x)
{
    float a = bf16_lo(w.x) * bf16_lo(x.x);
    a = __builtin_fmaf(bf16_hi(w.x), bf16_hi(x.x), a);
    a = __builtin_fmaf(bf16_lo(w.y), bf16_lo(x.y), a);
    a = __builtin_fmaf(bf16_hi(w.y), bf16_hi(x.y), a);
    a = __builtin_fmaf(bf16_lo(w.z), bf16_lo(x.z), a);
    a = __builtin_fmaf(bf16_hi(w.z), bf16_hi(x.z), a);
    a = __builtin_fmaf(bf16_lo(w.w), bf16_lo(x.w), a);
    a = __builtin_fmaf(bf16_hi(w.w), bf16_hi(x.w), a);
    return a;
}

// cols must be a multiple of 8 (16-byte pieces); checked on the host.
__global__ __launch_bounds__(64 * kWaves) void gemv_bf16_kernel(const uint16_t *__restrict__ W,
                                                               const uint16_t *__restrict__ x,
                                                               uint16_t *__restrict__ y, int rows,
                                                               int cols)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const v4u *wr = reinterpret_cast<const v4u *>(W + (size_t)row * cols);
    const v4u *xv = reinterpret_cast<const v4u *>(x);
    const int pieces = cols / 8;
    float acc = 0.f;
    int p = lane;
    for (; p + 3 * 64 < pieces; p += 4 * 64) {       // four 1 KiB loads in flight per lane group
        const v4u w0 = __builtin_nontemporal_load(wr + p);
        const v4u w1 = __builtin_nontemporal_load(wr + p + 64);
        const v4u w2 = __builtin_nontemporal_load(wr + p + 128);
        const v4u w3 = __builtin_nontemporal_load(wr + p + 192);
        acc += dot8(w0, xv[p]) + dot8(w1, xv[p + 64]) + dot8(w2, xv[p + 128]) + dot8(w3, xv[p + 192]);
    }
    for (; p < pieces; p += 64)
        acc += dot8(__builtin_nontemporal_load(wr + p), xv[p]);
    for (int off = 32; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off, 64);
    if (lane == 0)
        y[row] = to_bf16(acc);
}

// The ALU-only stand-in for a decode kernel: every thread runs `iters`
// dependent fused multiply-adds on registers and each workgroup stores one
// value at the end, so the kernel touches memory only in its last store.
// It tells waits in a kernel's own memory accesses apart from waits that any
// kernel sees (its dispatch and its end).
__global__ __launch_bounds__(64 * kWaves) void alu_kernel(float *__restrict__ out, int iters,
                                                         float seed)
{
    float a = seed + (float)threadIdx.x, b = 1.0f + 1e-7f * (float)blockIdx.x;
    for (int i = 0; i < iters; ++i)
        a = __builtin_fmaf(a, b, 1e-7f);
    a += __shfl_xor(a, 1, 64);
    if (threadIdx.x == 0)
        out[blockIdx.x & 1023] = a;
}

// A kernel that does nothing: its duration from the kernel's own events is
// the launch floor of a grid of that shape.
__global__ __launch_bounds__(64 * kWaves) void empty_kernel() {}

}  // namespace

extern "C" {

// A chain of n ALU-only kernels of `grid` workgroups and `iters` dependent
// FMAs per thread on `stream`; `out` holds at least 1,024 floats.  Returns a
// hipError_t value.
int kvload_alu_chain(float *out, int n, int grid, int iters, hipStream_t stream)
{
    if (!out || n <= 0 || grid <= 0 || grid > (1 << 20) || iters <= 0)
        return (int)hipErrorInvalidValue;
    for (int i = 0; i < n; ++i) {
        hipLaunchKernelGGL(alu_kernel, dim3(grid), dim3(64 * kWaves), 0, stream, out, iters,
                           (float)i);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return (int)e;
    }
    return 0;
}

// One empty kernel of `grid` workgroups of 256 threads; `start` and `stop`
// (either may be null) are recorded at the kernel's own start and end.
int kvload_empty(int grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    if (grid <= 0 || grid > (1 << 22))
        return (int)hipErrorInvalidValue;
    return (int)hipExtLaunchKernel(reinterpret_cast<const void *>(&empty_kernel), dim3(grid),
                                   dim3(64 * kWaves), nullptr, 0, stream, start, stop, 0);
}

// One product on `stream`.  Returns a hipError_t value (0 on success);
// hipErrorInvalidValue for non-positive sizes or cols not a multiple of 8.
int kvload_gemv_bf16(const void *W, const void *x, void *y, int rows, int cols, hipStream_t stream)
{
    if (rows <= 0 || cols <= 0 || (cols & 7) || !W || !x || !y)
        return (int)hipErrorInvalidValue;
    const dim3 grid((rows + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(gemv_bf16_kernel, grid, dim3(64 * kWaves), 0, stream,
                       (const uint16_t *)W, (const uint16_t *)x, (uint16_t *)y, rows, cols);
    return (int)hipGetLastError();
}

// A decode step: n products, product i uses weights Ws[i] of shape
// [rows[i], cols[i]] and reads the previous product's output (acts[i] ->
// acts[i + 1]).  acts has n + 1 device buffers.
int kvload_chain_bf16(const void *const *Ws, const int *rows, const int *cols, void *const *acts,
                      int n, hipStream_t stream)
{
    for (int i = 0; i < n; ++i) {
        const int rc = kvload_gemv_bf16(Ws[i], acts[i], acts[i + 1], rows[i], cols[i], stream);
        if (rc != 0)
            return rc;
    }
    return 0;
}

}  // extern "C"
