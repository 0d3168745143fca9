// runtime.cpp -- kvcopy_batch: staging, launch, errors; host allocation helpers.
//
// A call plans the batch straight into a library-owned pinned staging ring
// (with non-temporal stores: only the GPU reads the records) and launches
// one copy kernel on the caller's stream (PegaFlow issue #408, "Summary":
// one descriptor upload and one copy-kernel launch per batch).  A batch of
// at most 128 chunks passes its worklist in the kernel arguments instead,
// and kvcopy_batch_pair plans two lists into one region for one kernel.
// The kernel reads its worklist in place from the pinned ring, over the host
// link, with vector loads of 64 records at a time: the worklist crosses the
// link once, as part of the kernel's own traffic, with no separate copy and
// no copy-engine latency in front of the kernel.  (KVCOPY_F_DESC_UPLOAD
// instead copies it into a device twin of the ring with hipMemcpyAsync on a
// stream of the library's own, which the caller's stream waits for; with
// KVCOPY_F_DST_ORDER two order kernels follow that copy on the same stream
// and group the records by destination region into the twin's second half.)
//
// The vLLM PR #42212 report, section "review highlights", points out that
// descriptor buffers must be pinned for the transfer to be asynchronous, and
// that they are allocated once and reused.  Here each device has one pinned
// ring, sized once (it grows only if a single call needs more than a quarter
// of it).  Each call takes the next free region of the ring; the region is
// released when the kernel's completion event (the stop event of its own
// launch) has fired.  A call waits on the host only when the ring is full of
// regions whose kernels are still running.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "kvcopy.h"
#include "kvcopy_internal.h"
#include "staging_ring.h"

namespace kvc {
namespace {

thread_local int t_last_hip_error = 0;

}  // namespace

int hip_fail(hipError_t e)
{
    t_last_hip_error = (int)e;
    return KVCOPY_EHIP;
}

namespace {

constexpr uint64_t kRingMinBytes = 16ull << 20;   // 16 MiB: ~700 K worklist records
constexpr uint64_t kAlign = 256;

// Event operations of the staging ring on HIP events.
struct HipEventOps {
    std::vector<hipEvent_t> *spare;   // completed events, reused by later calls
    int poll(hipEvent_t e)
    {
        const hipError_t r = hipEventQuery(e);
        if (r == hipErrorNotReady)
            return 0;
        return r == hipSuccess ? 1 : hip_fail(r);
    }
    int wait(hipEvent_t e)
    {
        const hipError_t r = hipEventSynchronize(e);
        return r == hipSuccess ? 0 : hip_fail(r);
    }
    void recycle(hipEvent_t e) { spare->push_back(e); }
};

struct Staging {
    std::mutex mu;             // held for a whole call: planning is host-side and short
    int tuned[3] = {-2, -2, -2};   // kvcopy_autotune's cap per direction (-2: not tuned)
    uint8_t *host = nullptr;   // pinned, mapped (device address == host address)
    uint8_t *dev = nullptr;    // device twin (two halves), allocated on first KVCOPY_F_DESC_UPLOAD
    // KVCOPY_F_DYNAMIC: one pair of claim counters (next chunk, wavefronts
    // done) per 256-byte granule of the ring, in device memory, allocated on
    // first use and zeroed once.  A call uses the pair of its region's first
    // granule, which no other region in flight shares; the call's last
    // wavefront resets the pair to zero.
    uint32_t *claims = nullptr;
    int clock_khz = 0;             // wall-clock rate (hipDeviceAttributeWallClockRate), 0 = not read yet
    std::vector<ChunkRec> order_tmp;   // KVCOPY_F_DST_ORDER: the worklist in list order
    // KVCOPY_F_DESC_UPLOAD: the worklist copies run on a stream of the
    // library's own (default priority), created on first use; the caller's
    // stream waits for each copy through `up_done` before its kernel.
    hipStream_t up_stream = nullptr;
    hipEvent_t up_done = nullptr;
    std::vector<hipEvent_t> spare;
    StagingRing<hipEvent_t, HipEventOps> ring{HipEventOps{&spare}};
};

std::mutex g_staging_mu;
std::vector<Staging *> g_staging;   // indexed by device ordinal; lives until process exit

Staging *staging_for(int device)
{
    std::lock_guard<std::mutex> g(g_staging_mu);
    if ((size_t)device >= g_staging.size())
        g_staging.resize((size_t)device + 1, nullptr);
    if (g_staging[device] == nullptr)
        g_staging[device] = new Staging();
    return g_staging[device];
}

// Makes the ring at least 4 x `need` bytes (and allocates the device twin if
// `want_dev`, the claim counters if `want_claims`).  Old buffers are
// released only after every kernel using them has completed.
int grow(Staging *st, uint64_t need, bool want_dev, bool want_claims)
{
    uint64_t cap = st->ring.capacity() ? st->ring.capacity() : kRingMinBytes;
    while (cap < 4 * need)
        cap *= 2;
    const bool resize = cap != st->ring.capacity();
    if (!resize && (!want_dev || st->dev) && (!want_claims || st->claims))
        return KVCOPY_OK;
    int rc = st->ring.drain();
    if (rc != KVCOPY_OK)
        return rc;
    // Work on the upload stream belongs to committed regions (drained above)
    // except after a call that failed between its upload and its kernel: let
    // that finish too before the buffers it uses are freed.
    if (st->up_stream != nullptr) {
        const hipError_t se = hipStreamSynchronize(st->up_stream);
        if (se != hipSuccess)
            return hip_fail(se);
    }
    if (resize) {
        if (st->host)
            (void)hipHostFree(st->host);
        if (st->dev)
            (void)hipFree(st->dev);
        if (st->claims) {
            want_claims = true;
            (void)hipFree(st->claims);
        }
        st->host = nullptr;
        st->dev = nullptr;
        st->claims = nullptr;
        st->ring.reset(0);
    }
    hipError_t e;
    if (st->host == nullptr) {
        e = hipHostMalloc((void **)&st->host, cap, hipHostMallocMapped | hipHostMallocPortable);
        if (e != hipSuccess) {
            st->host = nullptr;
            return e == hipErrorOutOfMemory ? KVCOPY_ENOMEM : hip_fail(e);
        }
        // Touch every page once now: measured on MI355X hosts, the first
        // pass of the planner over fresh ring pages ran at about 2 GB/s (690
        // us per 65,536-record worklist, against 100-150 us once the ring had
        // wrapped), which made the first ten or so large calls host-bound.
        memset(st->host, 0, cap);
    }
    st->ring.reset(cap);
    if (want_dev && st->dev == nullptr) {
        // two halves: the uploaded regions, and at the same offsets in the
        // second half their destination-ordered copies (launch_order)
        e = hipMalloc((void **)&st->dev, 2 * cap);
        if (e != hipSuccess) {
            st->dev = nullptr;
            return e == hipErrorOutOfMemory ? KVCOPY_ENOMEM : hip_fail(e);
        }
    }
    if (want_claims && st->claims == nullptr) {
        const uint64_t bytes = cap / kAlign * 2 * sizeof(uint32_t);
        e = hipMalloc((void **)&st->claims, bytes);
        if (e != hipSuccess) {
            st->claims = nullptr;
            return e == hipErrorOutOfMemory ? KVCOPY_ENOMEM : hip_fail(e);
        }
        // Once, at allocation (the ring is drained): from here on every
        // kernel leaves its pair at zero.
        if ((e = hipMemset(st->claims, 0, bytes)) != hipSuccess) {
            (void)hipFree(st->claims);
            st->claims = nullptr;
            return hip_fail(e);
        }
    }
    return KVCOPY_OK;
}

// KVCOPY_WGS_AUTO: the tuned cap if the device was probed, else the fixed
// defaults measured on MI355X (128 for the host-link directions, the full
// grid for D2D).
int resolve_auto(const Staging *st, int dir)
{
    if (st->tuned[dir] >= 0)
        return st->tuned[dir];
    return dir == KVCOPY_D2D ? KVCOPY_WGS_ALL : 128;
}

// KVCOPY_WGS_AUTO for kvcopy_batch_pair: with 16,384 x 4 KiB each way, one
// launch measured 98.4 GB/s on MI355X at 64 workgroups with no slow window
// in 30; 96-160 workgroups reached 99.1-99.5 GB/s at the median but had
// occasional windows below 50 GB/s, and 48 gave 97.9.
constexpr int kPairAutoWgs = 64;

// KVCOPY_F_TAIL_BOUNDED: measured on MI355X (a bf16 GEMV decode loop beside
// H2D + D2H bursts of 16,384 x 4 KiB every 50 ms): 4 workgroups per stream
// issuing in 2 us of every 20 us with sc1 stores held the decode's p99 to
// +4.9% and its worst step to 0.44 ms (0.41 ms alone); a 40 us period gave
// +2.8% and 0.41 ms at half the transfer rate, 8 workgroups +6.1% / 0.43 ms.
constexpr uint32_t kTailDutyOnNs = 2000, kTailDutyPeriodNs = 20000;
constexpr int kTailMaxWgs = 4;

// The per-call options after parsing.
struct CallOpts {
    uint32_t chunk = KVCOPY_CHUNK_DEFAULT;
    uint32_t flags = 0;
    uint32_t duty_on_ns = 0, duty_period_ns = 0;   // period 0: no pacing
    hipEvent_t ev_begin = nullptr, ev_end = nullptr;
};

// KVCOPY_F_STORE_SC1 / KVCOPY_F_STORE_NT: -1 when neither is given.
int forced_store(uint32_t flags)
{
    if (flags & KVCOPY_F_STORE_SC1)
        return 1;
    if (flags & KVCOPY_F_STORE_NT)
        return 0;
    return -1;
}

// Duty cycle in wall-clock ticks of `device` (read once per device).
int pace_ticks(Staging *st, int device, const CallOpts &o, uint32_t *on, uint32_t *period)
{
    *on = *period = 0;
    if (o.duty_period_ns == 0 || o.duty_on_ns == o.duty_period_ns)
        return KVCOPY_OK;
    if (st->clock_khz == 0) {
        int khz = 0;
        const hipError_t e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device);
        if (e != hipSuccess)
            return hip_fail(e);
        if (khz <= 0)
            return hip_fail(hipErrorInvalidValue);
        st->clock_khz = khz;
    }
    // ticks = ns * kHz / 1e6, the window rounded up and the period down, at
    // least 100 ticks on (the kernel polls the clock every few ticks)
    const uint64_t k = (uint64_t)st->clock_khz;
    uint64_t t_on = ((uint64_t)o.duty_on_ns * k + 999999) / 1000000;
    uint64_t t_per = (uint64_t)o.duty_period_ns * k / 1000000;
    if (t_on < 100)
        t_on = 100;
    if (t_per > 1000000)
        t_per = 1000000;
    if (t_on >= t_per)
        return KVCOPY_OK;   // the window covers the period: no pacing
    *on = (uint32_t)t_on;
    *period = (uint32_t)t_per;
    return KVCOPY_OK;
}

// Plans the batch into the staging ring and enqueues the kernel (and, with
// KVCOPY_F_DESC_UPLOAD, the worklist copy before it).  Called with st->mu
// held.  One checked pass validates the list and writes its worklist into a
// region sized for `hint` records (twice the descriptor count, or the exact
// chunk count when known); only a batch with more chunks than that (many
// ranges longer than two chunks) is planned a second time into a region of
// the exact size.
int run_locked(Staging *st, int device, const uint64_t *src, const uint64_t *dst,
               const uint64_t *sizes, uint64_t n, uint64_t hint, int dir, int max_wgs,
               hipStream_t stream, const CallOpts &o)
{
    const uint32_t flags = o.flags, chunk = o.chunk;
    const bool upload = (flags & KVCOPY_F_DESC_UPLOAD) != 0;
    const bool dynamic = (flags & KVCOPY_F_DYNAMIC) != 0;
    const bool merge = !(flags & KVCOPY_F_NO_COALESCE);
    const bool dst_order = (flags & KVCOPY_F_DST_ORDER) != 0;
    // Destination order of an uploaded worklist is made on the GPU
    // (launch_order): the region starts with the order kernels' zeroed
    // header, and the records follow it.
    const bool gpu_order = dst_order && upload;
    const uint64_t head = gpu_order ? kOrderHeaderBytes : 0;
    uint32_t pace_on = 0, pace_period = 0;
    int rc = pace_ticks(st, device, o, &pace_on, &pace_period);
    if (rc != KVCOPY_OK)
        return rc;
    uint64_t off = 0, n_chunks = 0;
    ChunkRec *host = nullptr;
    if (dst_order && !upload) {
        // Plan in list order into host memory of the library's own, then
        // place the records into the ring in destination order.
        std::vector<ChunkRec> &tmp = st->order_tmp;
        for (int pass = 0; pass < 2; ++pass) {
            const uint64_t room = hint ? hint : 1;
            try {
                if (tmp.size() < room)
                    tmp.resize(room);
            } catch (...) {
                return KVCOPY_ENOMEM;
            }
            if ((rc = build_checked(src, dst, sizes, n, merge, chunk, tmp.data(), room,
                                    &n_chunks)) != KVCOPY_OK)
                return rc;
            if (n_chunks == 0)
                return KVCOPY_OK;   // only zero-size descriptors: nothing to enqueue
            if (n_chunks > KVCOPY_MAX_CHUNKS)
                return KVCOPY_EINVAL;
            if (n_chunks <= room)
                break;
            hint = n_chunks;   // plan again with room for every record
        }
        const uint64_t need = (n_chunks * sizeof(ChunkRec) + kAlign - 1) / kAlign * kAlign;
        if (4 * need > st->ring.capacity() || (upload && st->dev == nullptr) ||
            (dynamic && st->claims == nullptr)) {
            if ((rc = grow(st, need, upload, dynamic)) != KVCOPY_OK)
                return rc;
        }
        if ((rc = st->ring.reserve(need, &off)) != KVCOPY_OK)
            return rc;
        host = reinterpret_cast<ChunkRec *>(st->host + off);
        order_by_dst(st->order_tmp.data(), n_chunks, host);
    } else {
        for (int pass = 0; pass < 2; ++pass) {
            const uint64_t room = hint ? hint : 1;
            const uint64_t need = (head + room * sizeof(ChunkRec) + kAlign - 1) / kAlign * kAlign;
            if (4 * need > st->ring.capacity() || (upload && st->dev == nullptr) ||
                (dynamic && st->claims == nullptr)) {
                if ((rc = grow(st, need, upload, dynamic)) != KVCOPY_OK)
                    return rc;
            }
            if ((rc = st->ring.reserve(need, &off)) != KVCOPY_OK)
                return rc;
            host = reinterpret_cast<ChunkRec *>(st->host + off + head);
            if ((rc = build_checked(src, dst, sizes, n, merge, chunk, host, room, &n_chunks,
                                    true)) != KVCOPY_OK)
                return rc;   // nothing committed: the region stays free
            if (n_chunks == 0)
                return KVCOPY_OK;   // only zero-size descriptors: nothing to enqueue
            if (n_chunks > KVCOPY_MAX_CHUNKS)
                return KVCOPY_EINVAL;
            if (n_chunks <= room)
                break;
            hint = n_chunks;   // plan again into a region of the exact size
        }
    }
    const uint64_t used = (head + n_chunks * sizeof(ChunkRec) + kAlign - 1) / kAlign * kAlign;
    if (gpu_order)
        memset(st->host + off, 0, head);
    finish_records();   // the streamed records reach memory before the launch is queued

    const ChunkRec *recs = host;   // read in place: mapped at the same address on the device
    hipError_t e;
    if (upload) {
        // The copy depends only on the host having written the region, so it
        // runs on the library's own stream and overlaps whatever the caller's
        // stream is still running (the previous call's kernel, in a train of
        // calls); the caller's stream waits for it before the kernel.  The
        // region's device twin is free: the ring hands a region out again
        // only after its last kernel, which waited for its copy, completed.
        if (st->up_stream == nullptr) {
            hipStream_t us = nullptr;
            hipEvent_t ue = nullptr;
            if ((e = hipStreamCreateWithFlags(&us, hipStreamNonBlocking)) != hipSuccess)
                return hip_fail(e);
            if ((e = hipEventCreateWithFlags(&ue, hipEventDisableTiming)) != hipSuccess) {
                (void)hipStreamDestroy(us);
                return hip_fail(e);
            }
            st->up_stream = us;   // both or neither
            st->up_done = ue;
        }
        if ((e = hipMemcpyAsync(st->dev + off, st->host + off, head + n_chunks * sizeof(ChunkRec),
                                hipMemcpyHostToDevice, st->up_stream)) != hipSuccess)
            return hip_fail(e);
        recs = reinterpret_cast<const ChunkRec *>(st->dev + off + head);
        if (gpu_order) {
            // The order kernels follow the copy on the same stream, so in a
            // train of calls they too overlap the previous call's kernel.
            // Their output goes to the second half of the device twin, at the
            // region's offset there.
            ChunkRec *ordered =
                reinterpret_cast<ChunkRec *>(st->dev + st->ring.capacity() + off + head);
            if ((e = launch_order(recs, (uint32_t)n_chunks, ordered,
                                  reinterpret_cast<uint32_t *>(st->dev + off), st->up_stream,
                                  nullptr)) != hipSuccess)
                return hip_fail(e);
            recs = ordered;
        }
        if ((e = hipEventRecord(st->up_done, st->up_stream)) != hipSuccess ||
            (e = hipStreamWaitEvent(stream, st->up_done, 0)) != hipSuccess)
            return hip_fail(e);
    }
    if (max_wgs == KVCOPY_WGS_AUTO)
        max_wgs = resolve_auto(st, dir);
    // The region's completion event is bound to the kernel itself (the stop
    // event of hipExtLaunchKernel): recording a separate event after the
    // kernel measured 4.3 us of extra GPU time per call on MI355X.  When the
    // caller asks for the kernel's own start and end (timing), those take
    // the launch's event slots and the completion event is recorded after
    // the kernel instead.
    const bool timed = o.ev_begin != nullptr || o.ev_end != nullptr;
    hipEvent_t done;
    if (!st->spare.empty()) {
        done = st->spare.back();
        st->spare.pop_back();
    } else if ((e = hipEventCreateWithFlags(&done, hipEventDisableTiming)) != hipSuccess) {
        return hip_fail(e);
    }
    const uint32_t grid = grid_for(n_chunks, max_wgs);
    hipEvent_t start = timed ? o.ev_begin : nullptr, stop = timed ? o.ev_end : done;
    if (flags & KVCOPY_F_WG_PER_CHUNK) {
        const uint32_t g = grid_for_wg(n_chunks, max_wgs);
        int sc1 = forced_store(flags);
        if (sc1 < 0)
            sc1 = default_sc1(dir, g);
        e = launch_copy_wg(recs, (uint32_t)n_chunks, g, dir, sc1 != 0, stream, start, stop);
    } else if (dynamic) {
        uint32_t *claim = st->claims + off / kAlign * 2;
        const uint32_t g = grid < kDynMaxGrid ? grid : kDynMaxGrid;
        e = launch_copy_dynamic(recs, (uint32_t)n_chunks, g, dir, claim, claim_grain(n_chunks, g),
                                stream, start, stop);
    } else {
        // A forced store form or pacing selects the per-chunk loop.
        const bool per_chunk = (flags & (KVCOPY_F_PER_CHUNK | KVCOPY_F_STORE_SC1 |
                                         KVCOPY_F_STORE_NT)) != 0 || pace_period != 0;
        const bool pipelined = (flags & KVCOPY_F_PIPELINE) != 0 ||
                               (!per_chunk && pipeline_pays(dir, grid, n_chunks));
        // D2H stores take the sc1 form on grids of three or more workgroups
        // and the other cases nt (copy_chunk.h, kSc1StorePolicy;
        // default_sc1), unless a flag forces one.  Only the speed depends on
        // the choice.
        int sc1 = forced_store(flags);
        if (sc1 < 0)
            sc1 = default_sc1(dir, grid);
        e = launch_copy(recs, (uint32_t)n_chunks, grid, dir, pipelined, sc1 != 0, pace_on,
                        pace_period, stream, start, stop);
    }
    if (e == hipSuccess && timed)
        e = hipEventRecord(done, stream);
    if (e != hipSuccess) {
        st->spare.push_back(done);
        return hip_fail(e);
    }
    st->ring.commit(off, used, done);
    return KVCOPY_OK;
}

constexpr int kNotInline = 1;   // run_inline's "use the staging ring instead"

// Small batches (at most kInlineRecs chunks): the worklist goes to the GPU in
// the kernel arguments, so the call needs no staging region and no
// completion event, and the kernel makes no round trip over the host link
// for its records.  Returns kNotInline, with *chunks set to the batch's
// chunk count, when the worklist does not fit or the default policy would
// pick the pipelined loop for this grid (small D2D grids).
int run_inline(Staging *st, const uint64_t *src, const uint64_t *dst, const uint64_t *sizes,
               uint64_t n, int dir, int max_wgs, hipStream_t stream, const CallOpts &o,
               uint64_t *chunks)
{
    InlineWork w;
    w.reserved = 0;
    uint64_t need = 0;
    const int rc = build_checked(src, dst, sizes, n, !(o.flags & KVCOPY_F_NO_COALESCE), o.chunk,
                                 w.rec, kInlineRecs, &need);
    if (rc != KVCOPY_OK)
        return rc;
    if (need == 0)
        return KVCOPY_OK;   // only zero-size descriptors: nothing to enqueue
    *chunks = need;
    if (need > kInlineRecs)
        return kNotInline;
    w.n_chunks = (uint32_t)need;
    if (max_wgs == KVCOPY_WGS_AUTO) {
        std::lock_guard<std::mutex> g(st->mu);
        max_wgs = resolve_auto(st, dir);
    }
    const uint32_t grid = grid_for(w.n_chunks, max_wgs);
    const int forced = forced_store(o.flags);
    if (!(o.flags & KVCOPY_F_PER_CHUNK) && forced < 0 && pipeline_pays(dir, grid, w.n_chunks))
        return kNotInline;
    const bool sc1 = forced < 0 ? default_sc1(dir, grid) : forced == 1;
    const hipError_t e = launch_copy_inline(w, grid, dir, sc1, stream, o.ev_begin, o.ev_end);
    return e == hipSuccess ? KVCOPY_OK : hip_fail(e);
}

// kvcopy_batch_pair under st->mu: both lists are planned into one staging
// region, list b's records right after list a's, and one kernel copies both.
int run_pair_locked(Staging *st, const uint64_t *const src[2], const uint64_t *const dst[2],
                    const uint64_t *const sizes[2], const uint64_t n[2], bool merge,
                    bool sc1_stores, int max_wgs, hipStream_t stream)
{
    uint64_t hint[2] = {2 * n[0], 2 * n[1]}, cnt[2] = {0, 0}, off = 0;
    ChunkRec *host = nullptr;
    int rc;
    for (int pass = 0; pass < 3; ++pass) {
        const uint64_t room = (hint[0] + hint[1]) ? hint[0] + hint[1] : 1;
        const uint64_t need = (room * sizeof(ChunkRec) + kAlign - 1) / kAlign * kAlign;
        if (4 * need > st->ring.capacity() && (rc = grow(st, need, false, false)) != KVCOPY_OK)
            return rc;
        if ((rc = st->ring.reserve(need, &off)) != KVCOPY_OK)
            return rc;
        host = reinterpret_cast<ChunkRec *>(st->host + off);
        if ((rc = build_checked(src[0], dst[0], sizes[0], n[0], merge, KVCOPY_CHUNK_DEFAULT, host,
                                room, &cnt[0], true)) != KVCOPY_OK)
            return rc;   // nothing committed: the region stays free
        const uint64_t room_b = cnt[0] <= room ? room - cnt[0] : 0;
        if ((rc = build_checked(src[1], dst[1], sizes[1], n[1], merge, KVCOPY_CHUNK_DEFAULT,
                                host + (cnt[0] <= room ? cnt[0] : 0), room_b, &cnt[1], true)) != KVCOPY_OK)
            return rc;
        if (cnt[0] + cnt[1] > KVCOPY_MAX_CHUNKS)
            return KVCOPY_EINVAL;
        if (cnt[0] + cnt[1] <= room)
            break;
        hint[0] = cnt[0];   // plan again into a region of the exact size
        hint[1] = cnt[1];
    }
    const uint64_t total = cnt[0] + cnt[1];
    if (total == 0)
        return KVCOPY_OK;   // only zero-size descriptors: nothing to enqueue
    finish_records();   // the streamed records reach memory before the launch is queued
    const uint64_t used = (total * sizeof(ChunkRec) + kAlign - 1) / kAlign * kAlign;
    if (max_wgs == KVCOPY_WGS_AUTO)
        max_wgs = kPairAutoWgs;
    hipError_t e;
    hipEvent_t done;
    if (!st->spare.empty()) {
        done = st->spare.back();
        st->spare.pop_back();
    } else if ((e = hipEventCreateWithFlags(&done, hipEventDisableTiming)) != hipSuccess) {
        return hip_fail(e);
    }
    e = launch_copy_pair(host, (uint32_t)cnt[0], host + cnt[0], (uint32_t)cnt[1],
                         grid_for(total, max_wgs), sc1_stores, stream, nullptr, done);
    if (e != hipSuccess) {
        st->spare.push_back(done);
        return hip_fail(e);
    }
    st->ring.commit(off, used, done);
    return KVCOPY_OK;
}

}  // namespace

void set_tuned_wgs(int device, int dir, int wgs)
{
    Staging *st = staging_for(device);
    std::lock_guard<std::mutex> g(st->mu);
    st->tuned[dir] = wgs;
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvcopy_batch_ex(const uint64_t *src_addrs, const uint64_t *dst_addrs,
                               const uint64_t *sizes, uint64_t n, int dir, int max_wgs,
                               hipStream_t stream, const kvcopy_opts_t *opts)
{
    CallOpts o;
    if (opts) {
        if (opts->struct_size != sizeof(kvcopy_opts_t) && opts->struct_size != KVCOPY_OPTS_V1_SIZE)
            return KVCOPY_EINVAL;
        if (opts->chunk_bytes) {
            if ((opts->chunk_bytes & 15u) || opts->chunk_bytes > KVCOPY_CHUNK_MAX)
                return KVCOPY_EINVAL;
            o.chunk = opts->chunk_bytes;
        }
        const uint32_t known = KVCOPY_F_VALIDATE | KVCOPY_F_NO_COALESCE | KVCOPY_F_DESC_UPLOAD |
                               KVCOPY_F_PIPELINE | KVCOPY_F_PER_CHUNK | KVCOPY_F_DYNAMIC |
                               KVCOPY_F_STORE_SC1 | KVCOPY_F_STORE_NT | KVCOPY_F_DST_ORDER |
                               KVCOPY_F_TAIL_BOUNDED | KVCOPY_F_WG_PER_CHUNK;
        if (opts->flags & ~known)
            return KVCOPY_EINVAL;
        const uint32_t loops = opts->flags & (KVCOPY_F_PIPELINE | KVCOPY_F_PER_CHUNK |
                                              KVCOPY_F_DYNAMIC | KVCOPY_F_WG_PER_CHUNK);
        if (loops & (loops - 1))   // more than one loop forced
            return KVCOPY_EINVAL;
        const uint32_t stores = opts->flags & (KVCOPY_F_STORE_SC1 | KVCOPY_F_STORE_NT);
        if (stores == (KVCOPY_F_STORE_SC1 | KVCOPY_F_STORE_NT) ||
            (stores && (opts->flags & (KVCOPY_F_PIPELINE | KVCOPY_F_DYNAMIC))))
            return KVCOPY_EINVAL;   // store forms exist for the per-chunk and workgroup loops
        if (opts->struct_size == sizeof(kvcopy_opts_t) && opts->duty_period_ns != 0) {
            if (opts->duty_on_ns < 1000 || opts->duty_on_ns > opts->duty_period_ns ||
                opts->duty_period_ns > 10000000u ||
                (opts->flags & (KVCOPY_F_PIPELINE | KVCOPY_F_DYNAMIC | KVCOPY_F_WG_PER_CHUNK)))
                return KVCOPY_EINVAL;
            o.duty_on_ns = opts->duty_on_ns;
            o.duty_period_ns = opts->duty_period_ns;
        }
        o.flags = opts->flags;
        o.ev_begin = opts->kernel_begin;
        o.ev_end = opts->kernel_end;
        if (o.flags & KVCOPY_F_TAIL_BOUNDED) {
            if (o.flags & (KVCOPY_F_PIPELINE | KVCOPY_F_DYNAMIC | KVCOPY_F_WG_PER_CHUNK))
                return KVCOPY_EINVAL;
            if (!(o.flags & KVCOPY_F_STORE_NT))
                o.flags |= KVCOPY_F_STORE_SC1;
            if (o.duty_period_ns == 0) {
                o.duty_on_ns = kTailDutyOnNs;
                o.duty_period_ns = kTailDutyPeriodNs;
            }
            if (max_wgs == KVCOPY_WGS_ALL || max_wgs == KVCOPY_WGS_AUTO || max_wgs > kTailMaxWgs)
                max_wgs = kTailMaxWgs;
        }
    }
    if (dir != KVCOPY_H2D && dir != KVCOPY_D2H && dir != KVCOPY_D2D)
        return KVCOPY_EINVAL;
    if (max_wgs < KVCOPY_WGS_AUTO || n > KVCOPY_MAX_DESCS)
        return KVCOPY_EINVAL;
    if (n == 0)
        return KVCOPY_OK;
    if (!src_addrs || !dst_addrs || !sizes)
        return KVCOPY_EINVAL;
    bool bad_env = false;
    const bool validate = env_validate(&bad_env) || (o.flags & KVCOPY_F_VALIDATE);
    if (bad_env)
        return KVCOPY_EINVAL;

    // Validation errors come back before anything is enqueued; the alignment
    // and range checks are part of the planning pass, except in validate
    // mode, where they run first so that they keep priority over the
    // overlap check.
    if (validate) {
        Prescan pre;
        int rc = prescan(src_addrs, dst_addrs, sizes, n, o.chunk, &pre);
        if (rc != KVCOPY_OK)
            return rc;
        if ((rc = check_overlap(src_addrs, dst_addrs, sizes, n)) != KVCOPY_OK)
            return rc;
    }

    int device = 0;
    const hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) {
        // Argument errors keep priority over a failing runtime.
        Prescan pre;
        const int rc = prescan(src_addrs, dst_addrs, sizes, n, o.chunk, &pre);
        if (rc != KVCOPY_OK)
            return rc;
        if (pre.bound > KVCOPY_MAX_CHUNKS)
            return KVCOPY_EINVAL;
        return pre.nnz == 0 ? KVCOPY_OK : hip_fail(e);
    }
    Staging *st = staging_for(device);
    // Room for the first planning pass: two records per descriptor covers
    // batches whose ranges are mostly up to two chunks long (mixed 4-28 KiB
    // sizes with 16 KiB chunks, say), so they are planned once; the region's
    // unused tail is not committed.
    uint64_t hint = n <= KVCOPY_MAX_DESCS / 2 ? 2 * n : n;
    const uint32_t ring_only = KVCOPY_F_DESC_UPLOAD | KVCOPY_F_PIPELINE | KVCOPY_F_DYNAMIC |
                               KVCOPY_F_DST_ORDER | KVCOPY_F_WG_PER_CHUNK;
    if (n <= kInlineRecs && !(o.flags & ring_only) && o.duty_period_ns == 0) {
        const int rc = run_inline(st, src_addrs, dst_addrs, sizes, n, dir, max_wgs, stream, o,
                                  &hint);
        if (rc != kNotInline)
            return rc;
    }
    std::lock_guard<std::mutex> g(st->mu);
    return run_locked(st, device, src_addrs, dst_addrs, sizes, n, hint, dir, max_wgs, stream, o);
}

extern "C" int kvcopy_batch_pair(const uint64_t *src_a, const uint64_t *dst_a,
                                 const uint64_t *sizes_a, uint64_t n_a, const uint64_t *src_b,
                                 const uint64_t *dst_b, const uint64_t *sizes_b, uint64_t n_b,
                                 int max_wgs, uint32_t flags, hipStream_t stream)
{
    if (max_wgs < KVCOPY_WGS_AUTO || n_a > KVCOPY_MAX_DESCS || n_b > KVCOPY_MAX_DESCS ||
        (flags & ~(KVCOPY_F_VALIDATE | KVCOPY_F_NO_COALESCE | KVCOPY_F_STORE_NT)) != 0)
        return KVCOPY_EINVAL;
    if ((n_a && (!src_a || !dst_a || !sizes_a)) || (n_b && (!src_b || !dst_b || !sizes_b)))
        return KVCOPY_EINVAL;
    if (n_a + n_b == 0)
        return KVCOPY_OK;
    const uint64_t *const src[2] = {src_a, src_b}, *const dst[2] = {dst_a, dst_b};
    const uint64_t *const sizes[2] = {sizes_a, sizes_b};
    const uint64_t n[2] = {n_a, n_b};
    bool bad_env = false;
    const bool validate = env_validate(&bad_env) || (flags & KVCOPY_F_VALIDATE) != 0;
    if (bad_env)
        return KVCOPY_EINVAL;
    if (validate) {   // the overlap rule spans both lists
        for (int k = 0; k < 2; ++k) {
            Prescan pre;
            const int rc = prescan(src[k], dst[k], sizes[k], n[k], KVCOPY_CHUNK_DEFAULT, &pre);
            if (rc != KVCOPY_OK)
                return rc;
        }
        std::vector<uint64_t> s(src_a, src_a + n_a), d(dst_a, dst_a + n_a), z(sizes_a, sizes_a + n_a);
        s.insert(s.end(), src_b, src_b + n_b);
        d.insert(d.end(), dst_b, dst_b + n_b);
        z.insert(z.end(), sizes_b, sizes_b + n_b);
        const int rc = check_overlap(s.data(), d.data(), z.data(), n_a + n_b);
        if (rc != KVCOPY_OK)
            return rc;
    }
    int device = 0;
    const hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) {
        uint64_t bound = 0, nnz = 0;
        for (int k = 0; k < 2; ++k) {   // argument errors keep priority over a failing runtime
            Prescan pre;
            const int rc = prescan(src[k], dst[k], sizes[k], n[k], KVCOPY_CHUNK_DEFAULT, &pre);
            if (rc != KVCOPY_OK)
                return rc;
            bound += pre.bound;
            nnz += pre.nnz;
        }
        if (bound > KVCOPY_MAX_CHUNKS)
            return KVCOPY_EINVAL;
        return nnz == 0 ? KVCOPY_OK : hip_fail(e);
    }
    Staging *st = staging_for(device);
    std::lock_guard<std::mutex> g(st->mu);
    return run_pair_locked(st, src, dst, sizes, n, !(flags & KVCOPY_F_NO_COALESCE),
                           !(flags & KVCOPY_F_STORE_NT), max_wgs, stream);
}

extern "C" uint64_t kvcopy_device_workspace_bytes(uint64_t max_n)
{
    return device_workspace_bytes(max_n);
}

namespace {

// Argument checks and grid of kvcopy_batch_device and its no-allocation
// variant (KVCOPY_OK, or the error; nothing enqueued on error).
int device_call_args(const uint64_t *d_src, const uint64_t *d_dst, const uint64_t *d_sizes,
                     const uint64_t *d_n, uint64_t max_n, int dir, int max_wgs,
                     uint32_t *chunk_bytes, uint32_t *grid)
{
    if (dir != KVCOPY_H2D && dir != KVCOPY_D2H && dir != KVCOPY_D2D)
        return KVCOPY_EINVAL;
    if (max_wgs < KVCOPY_WGS_AUTO || max_n > KVCOPY_MAX_DESCS)
        return KVCOPY_EINVAL;
    if (*chunk_bytes == 0)
        *chunk_bytes = KVCOPY_CHUNK_DEFAULT;
    if ((*chunk_bytes & 15u) || *chunk_bytes > KVCOPY_CHUNK_MAX)
        return KVCOPY_EINVAL;
    if (max_n == 0)
        return KVCOPY_OK;
    if (!d_src || !d_dst || !d_sizes || !d_n)
        return KVCOPY_EINVAL;
    if (max_wgs == KVCOPY_WGS_AUTO) {
        int device = 0;
        const hipError_t e = hipGetDevice(&device);
        if (e != hipSuccess)
            return hip_fail(e);
        Staging *st = staging_for(device);
        std::lock_guard<std::mutex> g(st->mu);
        max_wgs = resolve_auto(st, dir);
    }
    *grid = max_wgs == 0 ? 1024u : (uint32_t)max_wgs < kMaxGrid ? (uint32_t)max_wgs : kMaxGrid;
    return KVCOPY_OK;
}

}  // namespace

extern "C" int kvcopy_batch_device(const uint64_t *d_src, const uint64_t *d_dst,
                                   const uint64_t *d_sizes, const uint64_t *d_n, uint64_t max_n,
                                   int dir, int max_wgs, uint32_t chunk_bytes, void *workspace,
                                   hipStream_t stream)
{
    uint32_t grid = 0;
    int rc = device_call_args(d_src, d_dst, d_sizes, d_n, max_n, dir, max_wgs, &chunk_bytes, &grid);
    if (rc != KVCOPY_OK || max_n == 0)
        return rc;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return KVCOPY_EINVAL;
    const hipError_t e = launch_device_batch(d_src, d_dst, d_sizes, d_n, max_n, chunk_bytes, grid,
                                             workspace, nullptr, stream);
    return e == hipSuccess ? KVCOPY_OK : hip_fail(e);
}

extern "C" int kvcopy_batch_device_noalloc(const uint64_t *d_src, const uint64_t *d_dst,
                                           const uint64_t *d_sizes, const uint64_t *d_n,
                                           uint64_t max_n, int dir, int max_wgs,
                                           uint32_t chunk_bytes, uint64_t *d_status,
                                           hipStream_t stream)
{
    if (max_n > KVCOPY_NOALLOC_MAX_N)
        return KVCOPY_EINVAL;
    uint32_t grid = 0;
    int rc = device_call_args(d_src, d_dst, d_sizes, d_n, max_n, dir, max_wgs, &chunk_bytes, &grid);
    if (rc != KVCOPY_OK || max_n == 0)
        return rc;
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return hip_fail(e);
    void *ws = nullptr;
    if ((e = noalloc_workspace(device, &ws)) != hipSuccess)
        return hip_fail(e);
    if (device_workspace_bytes(max_n) > noalloc_workspace_bytes())
        return KVCOPY_EINVAL;   // cannot happen for max_n <= KVCOPY_NOALLOC_MAX_N
    e = launch_device_batch(d_src, d_dst, d_sizes, d_n, max_n, chunk_bytes, grid, ws, d_status,
                            stream);
    return e == hipSuccess ? KVCOPY_OK : hip_fail(e);
}

extern "C" int kvcopy_batch(const uint64_t *src_addrs, const uint64_t *dst_addrs,
                            const uint64_t *sizes, uint64_t n, int dir, int max_wgs,
                            hipStream_t stream)
{
    return kvcopy_batch_ex(src_addrs, dst_addrs, sizes, n, dir, max_wgs, stream, nullptr);
}

extern "C" const char *kvcopy_strerror(int code)
{
    switch (code) {
    case KVCOPY_OK: return "success";
    case KVCOPY_EINVAL: return "invalid argument";
    case KVCOPY_EALIGN: return "address or size not a multiple of 8 bytes";
    case KVCOPY_EOVERLAP: return "destination ranges overlap each other or a source";
    case KVCOPY_ENOMEM: return "out of memory";
    case KVCOPY_EHIP: return "HIP call failed (see kvcopy_last_hip_error)";
    default: return "unknown status";
    }
}

extern "C" int kvcopy_last_hip_error(void)
{
    return t_last_hip_error;
}

extern "C" int kvcopy_host_alloc_mapped(uint64_t bytes, void **out)
{
    if (bytes == 0 || out == nullptr)
        return KVCOPY_EINVAL;
    *out = nullptr;
    void *p = nullptr;
    hipError_t e = hipHostMalloc(&p, (size_t)bytes, hipHostMallocMapped | hipHostMallocPortable);
    if (e == hipErrorOutOfMemory)
        return KVCOPY_ENOMEM;
    if (e != hipSuccess)
        return hip_fail(e);
    void *dp = nullptr;
    e = hipHostGetDevicePointer(&dp, p, 0);
    if (e != hipSuccess || dp != p) {
        (void)hipHostFree(p);
        return hip_fail(e != hipSuccess ? e : hipErrorInvalidValue);
    }
    *out = p;
    return KVCOPY_OK;
}

extern "C" int kvcopy_host_free(void *p)
{
    if (p == nullptr)
        return KVCOPY_OK;
    hipError_t e = hipHostFree(p);
    return e == hipSuccess ? KVCOPY_OK : hip_fail(e);
}
