// latency_tool.cpp -- per-call latency of kvcopy_batch seen from a C caller
// (measurement only; built next to libkvcopy.so as block_copy_amd/kvcopy_latency).
//
// The per-call figures that bench.py takes from Python include the
// binding's argument marshalling.  This program makes the same calls from
// C++, in a process without torch, so the library's own cost is visible:
//
//   kvcopy_latency FILE...
//
// Each FILE describes one batch (written by bench.py from its workloads):
//   char name[64]; uint32 src_host, dst_host; int32 max_wgs; uint32 flags;
//   uint64 src_bytes, dst_bytes, n;  uint64 src_off[n], dst_off[n], size[n]
// (offsets into a source and a destination arena; an arena is device memory
// from hipMalloc or mapped pinned host memory from kvcopy_host_alloc_mapped).
// For each file it times, on one stream:
//   host_us  the call's own time (return of kvcopy_batch), isolated calls;
//   wall_us  call + hipStreamSynchronize, isolated calls;
//   gpu_us   between events recorded on the stream before and after the call;
//   pipelined_us  back-to-back calls with no sync in between, per call
//            (after 50 untimed ones; at least 20 ms of calls);
// then checks that every destination range holds its source bytes, and
// prints one JSON object per file on stdout.  With the header flag bit
// kRuntimeCopy the calls are one hipMemcpyAsync per descriptor instead.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "kvcopy.h"

namespace {

struct Header {
    char name[64];
    uint32_t src_host, dst_host;
    int32_t max_wgs;
    uint32_t flags;   // KVCOPY_F_* for kvcopy_batch_ex (0: plain kvcopy_batch)
    uint64_t src_bytes, dst_bytes, n;
};

// A header flag bit outside the library's flags: time one hipMemcpyAsync per
// descriptor instead of kvcopy_batch (the runtime's copy, also from C).
constexpr uint32_t kRuntimeCopy = 0x80000000u;

bool ok(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return e == hipSuccess;
}

double now_us()
{
    return std::chrono::duration<double, std::micro>(
               std::chrono::steady_clock::now().time_since_epoch())
        .count();
}

double pct(std::vector<double> v, double q)
{
    std::sort(v.begin(), v.end());
    const size_t i = (size_t)(q / 100.0 * (double)(v.size() - 1) + 0.5);
    return v[std::min(i, v.size() - 1)];
}

uint64_t splitmix64(uint64_t *s)
{
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

struct Arena {
    uint8_t *p = nullptr;
    uint64_t bytes = 0;
    bool host = false;
    ~Arena()
    {
        if (p && host)
            kvcopy_host_free(p);
        else if (p)
            (void)hipFree(p);
    }
    bool alloc(uint64_t n, bool on_host)
    {
        bytes = n;
        host = on_host;
        if (host)
            return kvcopy_host_alloc_mapped(n, (void **)&p) == KVCOPY_OK;
        return ok(hipMalloc((void **)&p, n), "hipMalloc");
    }
    bool fill(uint8_t byte, uint64_t seed)   // seed 0: the byte; else pseudo-random
    {
        std::vector<uint8_t> img(bytes, byte);
        if (seed)
            for (uint64_t i = 0; i + 8 <= bytes; i += 8) {
                const uint64_t w = splitmix64(&seed);
                memcpy(img.data() + i, &w, 8);
            }
        if (host) {
            memcpy(p, img.data(), bytes);
            return true;
        }
        return ok(hipMemcpy(p, img.data(), bytes, hipMemcpyHostToDevice), "hipMemcpy");
    }
    bool image(std::vector<uint8_t> *out) const
    {
        out->resize(bytes);
        if (host) {
            memcpy(out->data(), p, bytes);
            return true;
        }
        return ok(hipMemcpy(out->data(), p, bytes, hipMemcpyDeviceToHost), "hipMemcpy");
    }
};

int run_file(const char *path, hipStream_t st)
{
    FILE *f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        return 1;
    }
    Header h;
    bool good = fread(&h, sizeof h, 1, f) == 1 && h.n > 0 && h.n <= KVCOPY_MAX_DESCS;
    std::vector<uint64_t> so, dof, sz;
    if (good) {
        so.resize(h.n);
        dof.resize(h.n);
        sz.resize(h.n);
        good = fread(so.data(), 8, h.n, f) == h.n && fread(dof.data(), 8, h.n, f) == h.n &&
               fread(sz.data(), 8, h.n, f) == h.n;
    }
    fclose(f);
    h.name[63] = 0;
    for (uint64_t i = 0; good && i < h.n; ++i)
        good = sz[i] <= h.src_bytes && so[i] <= h.src_bytes - sz[i] && sz[i] <= h.dst_bytes &&
               dof[i] <= h.dst_bytes - sz[i];
    if (!good) {
        fprintf(stderr, "%s: malformed batch file\n", path);
        return 1;
    }
    const int dir = h.src_host ? KVCOPY_H2D : h.dst_host ? KVCOPY_D2H : KVCOPY_D2D;
    Arena src, dst;
    if (!src.alloc(h.src_bytes, h.src_host) || !dst.alloc(h.dst_bytes, h.dst_host) ||
        !src.fill(0, 12345) || !dst.fill(0xA5, 0))
        return 1;
    std::vector<uint64_t> s(h.n), d(h.n);
    for (uint64_t i = 0; i < h.n; ++i) {
        s[i] = (uint64_t)(uintptr_t)src.p + so[i];
        d[i] = (uint64_t)(uintptr_t)dst.p + dof[i];
    }
    hipEvent_t e0, e1;
    if (!ok(hipEventCreate(&e0), "hipEventCreate") || !ok(hipEventCreate(&e1), "hipEventCreate"))
        return 1;
    kvcopy_opts_t opts;
    memset(&opts, 0, sizeof(opts));
    opts.struct_size = sizeof(opts);
    const bool runtime_copy = (h.flags & kRuntimeCopy) != 0;
    opts.flags = h.flags & ~kRuntimeCopy;
    const hipMemcpyKind kind = dir == KVCOPY_H2D   ? hipMemcpyHostToDevice
                               : dir == KVCOPY_D2H ? hipMemcpyDeviceToHost
                                                   : hipMemcpyDeviceToDevice;
    auto call = [&]() {
        if (runtime_copy) {
            for (uint64_t i = 0; i < h.n; ++i)
                if (!ok(hipMemcpyAsync(reinterpret_cast<void *>(d[i]),
                                       reinterpret_cast<const void *>(s[i]), sz[i], kind, st),
                        "hipMemcpyAsync"))
                    return false;
            return true;
        }
        const int rc = opts.flags ? kvcopy_batch_ex(s.data(), d.data(), sz.data(), h.n, dir,
                                                    h.max_wgs, st, &opts)
                                  : kvcopy_batch(s.data(), d.data(), sz.data(), h.n, dir, h.max_wgs, st);
        if (rc != KVCOPY_OK)
            fprintf(stderr, "kvcopy_batch: %s\n", kvcopy_strerror(rc));
        return rc == KVCOPY_OK;
    };
    uint64_t bytes = 0;
    for (uint64_t z : sz)
        bytes += z;
    // isolated calls: 20 to 300, about half a second of copying at 56 GB/s
    const int reps = (int)std::max<uint64_t>(20, std::min<uint64_t>(300, 28000000000ull / (bytes + 1)));
    std::vector<double> host_us, wall_us, gpu_us;
    for (int i = 0; i < reps + 10; ++i) {
        if (!ok(hipStreamSynchronize(st), "hipStreamSynchronize"))
            return 1;
        const double t0 = now_us();
        if (!call())
            return 1;
        const double t1 = now_us();
        if (!ok(hipStreamSynchronize(st), "hipStreamSynchronize"))
            return 1;
        const double t2 = now_us();
        if (i >= 10) {
            host_us.push_back(t1 - t0);
            wall_us.push_back(t2 - t0);
        }
    }
    for (int i = 0; i < reps + 5; ++i) {
        if (!ok(hipEventRecord(e0, st), "hipEventRecord") || !call() ||
            !ok(hipEventRecord(e1, st), "hipEventRecord") || !ok(hipEventSynchronize(e1), "sync"))
            return 1;
        float ms = 0;
        if (!ok(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime"))
            return 1;
        if (i >= 5)
            gpu_us.push_back(ms * 1e3);
    }
    // back-to-back calls: 50 untimed, then at least `reps` calls and at
    // least 20 ms of submissions (a few hundred 5 us calls alone would be
    // too short a window to time)
    for (int i = 0; i < 50; ++i)
        if (!call())
            return 1;
    if (!ok(hipStreamSynchronize(st), "hipStreamSynchronize"))
        return 1;
    const double t0 = now_us();
    int bb = 0;
    while (bb < reps || now_us() - t0 < 20000.0) {
        if (!call())
            return 1;
        ++bb;
    }
    if (!ok(hipStreamSynchronize(st), "hipStreamSynchronize"))
        return 1;
    const double pipelined = (now_us() - t0) / bb;
    // every destination range must hold its source bytes
    std::vector<uint8_t> si, di;
    if (!src.image(&si) || !dst.image(&di))
        return 1;
    uint64_t bad = 0;
    for (uint64_t i = 0; i < h.n; ++i)
        bad += memcmp(si.data() + so[i], di.data() + dof[i], sz[i]) != 0;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    printf("{\"name\": \"%s\", \"call\": \"%s\", \"descriptors\": %llu, \"bytes\": %llu, \"max_wgs\": %d, "
           "\"calls\": %d, \"host_us_p50\": %.2f, \"host_us_p99\": %.2f, \"wall_us_p50\": %.2f, "
           "\"wall_us_p99\": %.2f, \"gpu_us_p50\": %.2f, \"gpu_us_p99\": %.2f, "
           "\"pipelined_us_per_call\": %.2f, \"pipelined_calls\": %d, \"ranges_checked\": %llu, "
           "\"ranges_wrong\": %llu}\n",
           h.name, runtime_copy ? "hipMemcpyAsync per range" : "kvcopy_batch",
           (unsigned long long)h.n, (unsigned long long)bytes, h.max_wgs, reps,
           pct(host_us, 50), pct(host_us, 99), pct(wall_us, 50), pct(wall_us, 99), pct(gpu_us, 50),
           pct(gpu_us, 99), pipelined, bb, (unsigned long long)h.n, (unsigned long long)bad);
    fflush(stdout);
    return bad ? 2 : 0;
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc < 2) {
        fprintf(stderr, "usage: kvcopy_latency BATCH_FILE...\n");
        return 1;
    }
    hipStream_t st;
    if (!ok(hipStreamCreate(&st), "hipStreamCreate"))
        return 1;
    int rc = 0;
    for (int i = 1; i < argc && rc == 0; ++i)
        rc = run_file(argv[i], st);
    (void)hipStreamDestroy(st);
    return rc;
}
