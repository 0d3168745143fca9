// autotune.cpp -- kvcopy_autotune: a startup probe for the workgroup cap.
//
// FreeToken issue #751, section "Proposal", question 1: pick the worker
// count from a small startup probe, aiming at bytes in flight rather than
// threads.  The vLLM PR #42212 report, section "key source snippet" (the
// tuned constants), keeps the smallest worker count within 5% of peak.  The
// probe times shuffled 4 KiB blocks at a ladder of caps and keeps the
// largest cap within 2% of the best rate (see the tie rule below).  For H2D
// and D2H both directions run together, which is how KV offload bursts
// arrive (PegaFlow issue #408, "Test setup": H2D and D2H concurrently on
// separate streams).
//
// Window length and tie rule, measured on MI355X over three processes for
// H2D + D2H on two streams: with 6 timed batches per cap the probe rated
// 32 or 64 workgroups best (79-85 GB/s against 79-80 at 128), but those
// caps ran 600-step bursts at 79-81 GB/s against 76-86 at 128.  With 24
// batches of 8,192 blocks and a 2% tie rule toward the smaller cap it
// still picked 32 in one run
// (84.1 GB/s against 85.7 at 128, inside the window-to-window spread),
// which then ran the burst 3% slower than 128.  So the probe now uses the
// workload's own batch shape (16,384 blocks of 4 KiB per direction) and
// joins the two directions at every step as a caller's burst does.  Unlike
// the vLLM report's rule it breaks near-ties toward the larger cap: a
// smaller grid does not protect co-running kernels on this part (they wait
// on queued host-link traffic, not on compute units), and the smallest
// grids that rate well in a probe are the ones whose rate later dips.
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "kvcopy.h"
#include "kvcopy_internal.h"

namespace {

constexpr uint64_t kBlocks = 16384;
constexpr uint64_t kBlock = 4096;
constexpr uint64_t kBytes = kBlocks * kBlock;   // 64 MiB per direction
constexpr int kWarm = 4;                         // untimed batches per cap
constexpr int kReps = 24;                        // timed batches per cap
constexpr int kSweeps = 3;                       // ascending, descending, ascending
const int kCaps[KVCOPY_AUTOTUNE_NCAPS] = KVCOPY_AUTOTUNE_CAPS;

uint64_t splitmix(uint64_t &s)
{
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Block offsets of `a` in shuffled order (Fisher-Yates).
std::vector<uint64_t> shuffled(uint64_t base, uint64_t seed)
{
    std::vector<uint64_t> v(kBlocks);
    for (uint64_t i = 0; i < kBlocks; ++i)
        v[i] = base + i * kBlock;
    for (uint64_t i = kBlocks - 1; i > 0; --i)
        std::swap(v[i], v[splitmix(seed) % (i + 1)]);
    return v;
}

struct Probe {
    void *host[2] = {nullptr, nullptr};
    void *dev[2] = {nullptr, nullptr};
    hipStream_t s[2] = {nullptr, nullptr};
    bool own[2] = {false, false};   // streams created here (destroyed at the end)
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    hipEvent_t mark[2] = {nullptr, nullptr};   // per-step join of the two streams
    ~Probe()
    {   // release path: failures here cannot be reported and change nothing
        for (hipStream_t x : s)
            if (x)
                (void)hipStreamSynchronize(x);
        for (void *p : host)
            if (p)
                (void)hipHostFree(p);
        for (void *p : dev)
            if (p)
                (void)hipFree(p);
        for (hipEvent_t e : ev)
            if (e)
                (void)hipEventDestroy(e);
        for (hipEvent_t e : mark)
            if (e)
                (void)hipEventDestroy(e);
        for (int i = 0; i < 2; ++i)
            if (own[i])
                (void)hipStreamDestroy(s[i]);
    }
};

}  // namespace

extern "C" int kvcopy_autotune(int dir, hipStream_t s0, hipStream_t s1, int *out_wgs,
                               double *out_rates)
{
    if (dir != KVCOPY_H2D && dir != KVCOPY_D2H && dir != KVCOPY_D2D)
        return KVCOPY_EINVAL;
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return kvc::hip_fail(e);
    Probe p;
    const bool d2d = dir == KVCOPY_D2D;
    for (int i = 0; i < 2; ++i) {
        if (!d2d && (e = hipHostMalloc(&p.host[i], kBytes, hipHostMallocMapped | hipHostMallocPortable)) !=
                        hipSuccess)
            return e == hipErrorOutOfMemory ? KVCOPY_ENOMEM : kvc::hip_fail(e);
        if ((e = hipMalloc(&p.dev[i], kBytes)) != hipSuccess)
            return e == hipErrorOutOfMemory ? KVCOPY_ENOMEM : kvc::hip_fail(e);
        const hipStream_t given = i == 0 ? s0 : s1;
        if (given) {
            p.s[i] = given;
        } else {
            if ((e = hipStreamCreateWithFlags(&p.s[i], hipStreamNonBlocking)) != hipSuccess)
                return kvc::hip_fail(e);
            p.own[i] = true;
        }
    }
    for (hipEvent_t &x : p.ev)
        if ((e = hipEventCreate(&x)) != hipSuccess)
            return kvc::hip_fail(e);
    for (hipEvent_t &x : p.mark)
        if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess)
            return kvc::hip_fail(e);

    // Batches: D2D dev0 -> dev1; otherwise H2D host0 -> dev0 and D2H dev1 -> host1.
    struct B {
        std::vector<uint64_t> src, dst, size;
        int dir;
    } b[2];
    const int nb = d2d ? 1 : 2;
    if (d2d) {
        b[0] = {shuffled((uint64_t)p.dev[0], 1), shuffled((uint64_t)p.dev[1], 2),
                std::vector<uint64_t>(kBlocks, kBlock), KVCOPY_D2D};
    } else {
        b[0] = {shuffled((uint64_t)p.host[0], 3), shuffled((uint64_t)p.dev[0], 4),
                std::vector<uint64_t>(kBlocks, kBlock), KVCOPY_H2D};
        b[1] = {shuffled((uint64_t)p.dev[1], 5), shuffled((uint64_t)p.host[1], 6),
                std::vector<uint64_t>(kBlocks, kBlock), KVCOPY_D2H};
    }

    // Each cap is timed in three sweeps (ascending, descending, ascending)
    // and keeps its median rate: neither one slow window (a fresh stream's
    // first batches, say) nor one lucky window decides.  Two kernels on two
    // streams can fall into a state where one direction starves the other;
    // measured on MI355X, a cap of 32 per direction gave 83 GB/s in its best
    // windows but 72 in a typical one, which the better of two windows hid.
    double rates[KVCOPY_AUTOTUNE_NCAPS][kSweeps] = {};
    const int ncaps = (int)(sizeof(kCaps) / sizeof(kCaps[0]));
    for (int k = 0; k < kSweeps * ncaps; ++k) {
        const int sweep = k / ncaps, pos = k % ncaps;
        const int c = sweep % 2 == 0 ? pos : ncaps - 1 - pos;
        for (int rep = -kWarm; rep < kReps; ++rep) {   // negative reps: warm-up, untimed
            if (rep == 0) {
                if ((e = hipEventRecord(p.ev[0], p.s[0])) != hipSuccess ||
                    (e = hipStreamWaitEvent(p.s[1], p.ev[0], 0)) != hipSuccess)
                    return kvc::hip_fail(e);
            }
            for (int j = 0; j < nb; ++j) {
                const int rc = kvcopy_batch(b[j].src.data(), b[j].dst.data(), b[j].size.data(),
                                            kBlocks, b[j].dir, kCaps[c], p.s[j]);
                if (rc != KVCOPY_OK)
                    return rc;
            }
            if (nb == 2) {   // the step ends when both directions are done
                if ((e = hipEventRecord(p.mark[0], p.s[0])) != hipSuccess ||
                    (e = hipEventRecord(p.mark[1], p.s[1])) != hipSuccess ||
                    (e = hipStreamWaitEvent(p.s[0], p.mark[1], 0)) != hipSuccess ||
                    (e = hipStreamWaitEvent(p.s[1], p.mark[0], 0)) != hipSuccess)
                    return kvc::hip_fail(e);
            }
        }
        if ((e = hipEventRecord(p.ev[1], p.s[0])) != hipSuccess ||
            (e = hipEventRecord(p.ev[2], p.s[1])) != hipSuccess ||
            (e = hipEventSynchronize(p.ev[1])) != hipSuccess ||
            (e = hipEventSynchronize(p.ev[2])) != hipSuccess)
            return kvc::hip_fail(e);
        float ms0 = 0, ms1 = 0;
        if ((e = hipEventElapsedTime(&ms0, p.ev[0], p.ev[1])) != hipSuccess ||
            (e = hipEventElapsedTime(&ms1, p.ev[0], p.ev[2])) != hipSuccess)
            return kvc::hip_fail(e);
        const double ms = std::max(ms0, nb == 2 ? ms1 : 0.0f);
        rates[c][sweep] = ms > 0 ? (double)(kBytes * nb * kReps) / (ms * 1e-3) : 0;
    }
    double rate[KVCOPY_AUTOTUNE_NCAPS] = {};
    int best_c = 0;
    for (int c = 0; c < ncaps; ++c) {
        double r[kSweeps];
        std::copy(rates[c], rates[c] + kSweeps, r);
        std::sort(r, r + kSweeps);
        rate[c] = r[kSweeps / 2];
        if (rate[c] > rate[best_c])
            best_c = c;
    }
    // Among the caps whose median is within 2% of the best one, the largest
    // (the ladder ascends, with 0 = the full grid last).  Near-ties go to
    // the larger grid: on MI355X with H2D + D2H on two streams, 8 and 64
    // workgroups per stream rated within 0.5-1.1% of each other in six
    // processes, but at 8 one process in three then ran 20-step windows of
    // the burst at 88-92 GB/s against 96-97, while 64 stayed within
    // 94.6-96.4.  A single slow sweep does not disqualify a cap: either
    // cap showed one now and then.
    int chosen = kCaps[best_c];
    for (int c = 0; c < ncaps; ++c)
        if (c == best_c || rate[c] >= 0.98 * rate[best_c])
            chosen = kCaps[c];
    if (d2d) {
        kvc::set_tuned_wgs(device, KVCOPY_D2D, chosen);
    } else {
        kvc::set_tuned_wgs(device, KVCOPY_H2D, chosen);
        kvc::set_tuned_wgs(device, KVCOPY_D2H, chosen);
    }
    if (out_wgs)
        *out_wgs = chosen;
    if (out_rates)
        for (int c = 0; c < KVCOPY_AUTOTUNE_NCAPS; ++c)
            out_rates[c] = rate[c];
    return KVCOPY_OK;
}
