// runtime.cpp -- kvcopy_batch: staging, launch, errors; host allocation helpers.
//
// A call plans the batch straight into a library-owned pinned staging ring
// and launches one copy kernel on the caller's stream (PegaFlow issue #408,
// "Summary": one descriptor upload and one copy-kernel launch per batch).
// The kernel reads its worklist in place from the pinned ring, over the host
// link, with vector loads of 64 records at a time: the worklist crosses the
// link once, as part of the kernel's own traffic, with no separate copy and
// no copy-engine latency in front of the kernel.  (KVCOPY_F_DESC_UPLOAD
// instead copies it into a device twin of the ring with hipMemcpyAsync on
// the caller's stream.)
//
// The vLLM PR #42212 report, section "review highlights", points out that
// descriptor buffers must be pinned for the transfer to be asynchronous, and
// that they are allocated once and reused.  Here each device has one pinned
// ring, sized once (it grows only if a single call needs more than a quarter
// of it).  Each call takes the next free region of the ring; the region is
// released when an event recorded after the call's kernel has completed.  A
// call waits on the host only when the ring is full of regions whose kernels
// are still running.
#include <stdlib.h>
#include <string.h>

#include <deque>
#include <mutex>
#include <vector>

#include "kvcopy.h"
#include "kvcopy_internal.h"

namespace kvc {
namespace {

thread_local int t_last_hip_error = 0;

int hip_fail(hipError_t e)
{
    t_last_hip_error = (int)e;
    return KVCOPY_EHIP;
}

constexpr uint64_t kRingMinBytes = 16ull << 20;   // 16 MiB: ~700 K worklist records
constexpr uint64_t kAlign = 256;

struct InFlight {
    uint64_t begin, end;   // byte range of the ring
    hipEvent_t done;       // recorded after the kernel that reads the range
};

struct Staging {
    std::mutex mu;             // held for a whole call: planning is host-side and short
    uint8_t *host = nullptr;   // pinned, mapped (device address == host address)
    uint8_t *dev = nullptr;    // device twin, allocated on first KVCOPY_F_DESC_UPLOAD
    uint64_t cap = 0;
    uint64_t head = 0;         // next free byte
    std::deque<InFlight> inflight;   // allocation order == ring order
    std::vector<hipEvent_t> spare;   // completed events, reused
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

// Retires the oldest in-flight region: waits for its kernel if `wait`, else
// only polls.  Returns 1 if retired, 0 if still running (poll), or an error.
int retire_front(Staging *st, bool wait)
{
    const InFlight f = st->inflight.front();
    const hipError_t e = wait ? hipEventSynchronize(f.done) : hipEventQuery(f.done);
    if (e == hipErrorNotReady)
        return 0;
    if (e != hipSuccess)
        return hip_fail(e);
    st->spare.push_back(f.done);
    st->inflight.pop_front();
    if (st->inflight.empty())
        st->head = 0;
    return 1;
}

int drain(Staging *st)
{
    while (!st->inflight.empty()) {
        const int rc = retire_front(st, true);
        if (rc < 0)
            return rc;
    }
    return KVCOPY_OK;
}

// Makes the ring at least 4 x `need` bytes (and allocates the device twin if
// `want_dev`).  Old buffers are released only after every kernel using them
// has completed.
int grow(Staging *st, uint64_t need, bool want_dev)
{
    uint64_t cap = st->cap ? st->cap : kRingMinBytes;
    while (cap < 4 * need)
        cap *= 2;
    const bool resize = cap != st->cap;
    if (!resize && (!want_dev || st->dev))
        return KVCOPY_OK;
    int rc = drain(st);
    if (rc != KVCOPY_OK)
        return rc;
    if (resize) {
        if (st->host)
            hipHostFree(st->host);
        if (st->dev)
            hipFree(st->dev);
        st->host = nullptr;
        st->dev = nullptr;
        st->cap = 0;
    }
    hipError_t e;
    if (st->host == nullptr) {
        e = hipHostMalloc((void **)&st->host, cap, hipHostMallocMapped | hipHostMallocPortable);
        if (e != hipSuccess) {
            st->host = nullptr;
            return e == hipErrorOutOfMemory ? KVCOPY_ENOMEM : hip_fail(e);
        }
    }
    if (want_dev && st->dev == nullptr) {
        e = hipMalloc((void **)&st->dev, cap);
        if (e != hipSuccess) {
            st->dev = nullptr;
            st->cap = cap;   // the host ring is valid
            return e == hipErrorOutOfMemory ? KVCOPY_ENOMEM : hip_fail(e);
        }
    }
    st->cap = cap;
    st->head = 0;
    return KVCOPY_OK;
}

// Reserves `need` bytes at the ring's head (wrapping to 0 when the end of the
// ring is too short), retiring completed regions and waiting for running
// ones only when they are in the way.  *off receives the region's start.
int reserve(Staging *st, uint64_t need, bool want_dev, uint64_t *off)
{
    if (4 * need > st->cap || (want_dev && st->dev == nullptr)) {
        const int rc = grow(st, need, want_dev);
        if (rc != KVCOPY_OK)
            return rc;
    }
    while (!st->inflight.empty()) {   // retire whatever has finished, without waiting
        const int rc = retire_front(st, false);
        if (rc < 0)
            return rc;
        if (rc == 0)
            break;
    }
    for (;;) {
        if (st->inflight.empty()) {
            *off = 0;
            return KVCOPY_OK;
        }
        const uint64_t head = st->head, tail = st->inflight.front().begin;
        if (head > tail) {          // used [tail, head): free [head, cap) and [0, tail)
            if (head + need <= st->cap) {
                *off = head;
                return KVCOPY_OK;
            }
            if (need <= tail) {
                *off = 0;
                return KVCOPY_OK;
            }
        } else if (head < tail) {   // used wraps: free [head, tail)
            if (head + need <= tail) {
                *off = head;
                return KVCOPY_OK;
            }
        }                           // head == tail: the ring is full
        const int rc = retire_front(st, true);
        if (rc < 0)
            return rc;
    }
}

uint32_t grid_for(uint64_t n_chunks, int max_wgs)
{
    const uint64_t full = (n_chunks + kWavesPerWG - 1) / kWavesPerWG;   // one wavefront per chunk
    if (max_wgs == KVCOPY_WGS_ALL || (uint64_t)max_wgs >= full)
        return (uint32_t)full;
    return (uint32_t)max_wgs;
}

// Plans the batch into the staging ring and enqueues the kernel (and, with
// KVCOPY_F_DESC_UPLOAD, the worklist copy before it).  Called with st->mu held.
int run_locked(Staging *st, const uint64_t *src, const uint64_t *dst, const uint64_t *sizes,
               uint64_t n, const Prescan &pre, int dir, int max_wgs, hipStream_t stream,
               uint32_t chunk, uint32_t flags, hipEvent_t ev_begin, hipEvent_t ev_end)
{
    const bool upload = (flags & KVCOPY_F_DESC_UPLOAD) != 0;
    const uint64_t need = (pre.bound * sizeof(ChunkRec) + kAlign - 1) / kAlign * kAlign;
    uint64_t off = 0;
    int rc = reserve(st, need, upload, &off);
    if (rc != KVCOPY_OK)
        return rc;
    ChunkRec *host = reinterpret_cast<ChunkRec *>(st->host + off);
    const uint64_t n_chunks =
        build_worklist(src, dst, sizes, n, !(flags & KVCOPY_F_NO_COALESCE), chunk, host);
    const uint64_t used = (n_chunks * sizeof(ChunkRec) + kAlign - 1) / kAlign * kAlign;

    const ChunkRec *recs = host;   // read in place: mapped at the same address on the device
    hipError_t e;
    if (upload) {
        ChunkRec *dev = reinterpret_cast<ChunkRec *>(st->dev + off);
        if ((e = hipMemcpyAsync(dev, host, n_chunks * sizeof(ChunkRec), hipMemcpyHostToDevice,
                                stream)) != hipSuccess)
            return hip_fail(e);
        recs = dev;
    }
    if (ev_begin && (e = hipEventRecord(ev_begin, stream)) != hipSuccess)
        return hip_fail(e);
    if ((e = launch_copy(recs, (uint32_t)n_chunks, grid_for(n_chunks, max_wgs), dir, stream)) !=
        hipSuccess)
        return hip_fail(e);
    if (ev_end && (e = hipEventRecord(ev_end, stream)) != hipSuccess)
        return hip_fail(e);
    hipEvent_t done;
    if (!st->spare.empty()) {
        done = st->spare.back();
        st->spare.pop_back();
    } else if ((e = hipEventCreateWithFlags(&done, hipEventDisableTiming)) != hipSuccess) {
        return hip_fail(e);
    }
    if ((e = hipEventRecord(done, stream)) != hipSuccess) {
        st->spare.push_back(done);
        return hip_fail(e);
    }
    st->inflight.push_back(InFlight{off, off + used, done});
    st->head = off + used;
    return KVCOPY_OK;
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" int kvcopy_batch_ex(const uint64_t *src_addrs, const uint64_t *dst_addrs,
                               const uint64_t *sizes, uint64_t n, int dir, int max_wgs,
                               hipStream_t stream, const kvcopy_opts_t *opts)
{
    uint32_t chunk = KVCOPY_CHUNK_DEFAULT, flags = 0;
    hipEvent_t ev_begin = nullptr, ev_end = nullptr;
    if (opts) {
        if (opts->struct_size != sizeof(kvcopy_opts_t))
            return KVCOPY_EINVAL;
        if (opts->chunk_bytes) {
            if ((opts->chunk_bytes & 15u) || opts->chunk_bytes > KVCOPY_CHUNK_MAX)
                return KVCOPY_EINVAL;
            chunk = opts->chunk_bytes;
        }
        if (opts->flags & ~(KVCOPY_F_VALIDATE | KVCOPY_F_NO_COALESCE | KVCOPY_F_DESC_UPLOAD))
            return KVCOPY_EINVAL;
        flags = opts->flags;
        ev_begin = opts->kernel_begin;
        ev_end = opts->kernel_end;
    }
    if (dir != KVCOPY_H2D && dir != KVCOPY_D2H && dir != KVCOPY_D2D)
        return KVCOPY_EINVAL;
    if (max_wgs < 0 || n > KVCOPY_MAX_DESCS)
        return KVCOPY_EINVAL;
    if (n == 0)
        return KVCOPY_OK;
    if (!src_addrs || !dst_addrs || !sizes)
        return KVCOPY_EINVAL;
    bool bad_env = false;
    const bool validate = env_validate(&bad_env) || (flags & KVCOPY_F_VALIDATE);
    if (bad_env)
        return KVCOPY_EINVAL;

    Prescan pre;
    int rc = prescan(src_addrs, dst_addrs, sizes, n, chunk, &pre);
    if (rc != KVCOPY_OK)
        return rc;
    if (pre.bound > KVCOPY_MAX_CHUNKS)
        return KVCOPY_EINVAL;
    if (validate && (rc = check_overlap(src_addrs, dst_addrs, sizes, n)) != KVCOPY_OK)
        return rc;
    if (pre.nnz == 0)
        return KVCOPY_OK;   // only zero-size descriptors: nothing to enqueue

    int device = 0;
    const hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return hip_fail(e);
    Staging *st = staging_for(device);
    std::lock_guard<std::mutex> g(st->mu);
    return run_locked(st, src_addrs, dst_addrs, sizes, n, pre, dir, max_wgs, stream, chunk, flags,
                      ev_begin, ev_end);
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
        hipHostFree(p);
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
