// runtime.cpp -- kvcopy_batch: staging, upload, launch, errors; host allocation helpers.
//
// A call plans the batch into a library-owned pinned staging slot, uploads
// the chunk worklist with one async copy on the caller's stream and launches
// one copy kernel on the same stream (PegaFlow issue #408, "Summary": one
// descriptor upload and one copy-kernel launch).  The vLLM PR #42212 report,
// section "review highlights", notes that descriptor buffers that are not
// pinned make the "async" upload synchronous, and that the buffers are
// allocated once and reused: here each device keeps a ring of pinned slots,
// each with a device-side twin and an event recorded after the kernel that
// last read it.  A slot is reused only after that event has completed, so a
// caller never waits on its own stream inside the call except when all
// slots are still in flight.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <thread>
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

constexpr int kSlotsPerDevice = 8;

struct Slot {
    ChunkRec *host = nullptr;  // pinned, mapped staging (device-readable at the same address)
    ChunkRec *dev = nullptr;   // device twin the worklist is uploaded to
    uint64_t cap = 0;          // capacity in records
    hipEvent_t done = nullptr; // recorded after the last kernel that read this slot
    hipEvent_t uploaded = nullptr;  // recorded on the upload stream after the worklist copy
    bool recorded = false;
    bool busy = false;         // owned by a call in progress
};

struct DeviceRing {
    std::mutex mu;
    Slot slots[kSlotsPerDevice];
    unsigned next = 0;
    hipStream_t upload = nullptr;   // library-owned, non-blocking, default priority
};

std::mutex g_rings_mu;
std::vector<DeviceRing *> g_rings;   // indexed by device ordinal; never freed

DeviceRing *ring_for(int device)
{
    std::lock_guard<std::mutex> g(g_rings_mu);
    if ((size_t)device >= g_rings.size())
        g_rings.resize((size_t)device + 1, nullptr);
    if (g_rings[device] == nullptr)
        g_rings[device] = new DeviceRing();
    return g_rings[device];
}

// The device's upload stream, created on first use (with that device current).
int upload_stream(DeviceRing *r, hipStream_t *out)
{
    std::lock_guard<std::mutex> g(r->mu);
    if (r->upload == nullptr) {
        hipError_t e = hipStreamCreateWithFlags(&r->upload, hipStreamNonBlocking);
        if (e != hipSuccess) {
            r->upload = nullptr;
            return hip_fail(e);
        }
    }
    *out = r->upload;
    return KVCOPY_OK;
}

// Takes the next slot that no other call holds.  Returns nullptr only if
// every slot is busy (more concurrent callers than slots); the caller retries.
Slot *acquire(DeviceRing *r)
{
    std::lock_guard<std::mutex> g(r->mu);
    for (int t = 0; t < kSlotsPerDevice; ++t) {
        Slot *s = &r->slots[(r->next + t) % kSlotsPerDevice];
        if (!s->busy) {
            s->busy = true;
            r->next = (r->next + t + 1) % kSlotsPerDevice;
            return s;
        }
    }
    return nullptr;
}

void release(DeviceRing *r, Slot *s)
{
    std::lock_guard<std::mutex> g(r->mu);
    s->busy = false;
}

// Grows the slot to hold `need` records.  The slot's previous GPU work has
// completed (its event was waited on), so the old buffers can go.
int reserve(Slot *s, uint64_t need)
{
    if (need <= s->cap)
        return KVCOPY_OK;
    uint64_t cap = s->cap ? s->cap : 4096;
    while (cap < need)
        cap *= 2;
    if (s->host) {
        hipHostFree(s->host);
        s->host = nullptr;
    }
    if (s->dev) {
        hipFree(s->dev);
        s->dev = nullptr;
    }
    s->cap = 0;
    const size_t bytes = (size_t)cap * sizeof(ChunkRec);
    hipError_t e = hipHostMalloc((void **)&s->host, bytes, hipHostMallocMapped | hipHostMallocPortable);
    if (e == hipErrorOutOfMemory)
        return KVCOPY_ENOMEM;
    if (e != hipSuccess)
        return hip_fail(e);
    e = hipMalloc((void **)&s->dev, bytes);
    if (e != hipSuccess) {
        hipHostFree(s->host);
        s->host = nullptr;
        return e == hipErrorOutOfMemory ? KVCOPY_ENOMEM : hip_fail(e);
    }
    s->cap = cap;
    return KVCOPY_OK;
}

uint32_t grid_for(uint64_t n_chunks, int max_wgs)
{
    const uint64_t full = (n_chunks + kWavesPerWG - 1) / kWavesPerWG;   // one wavefront per chunk
    if (max_wgs == KVCOPY_WGS_ALL || (uint64_t)max_wgs >= full)
        return (uint32_t)full;
    return (uint32_t)max_wgs;
}

// Plans the batch straight into the slot's pinned staging, then enqueues the
// worklist upload and the kernel.  The slot is held by this call.
int run_in_slot(Slot *s, const uint64_t *src, const uint64_t *dst, const uint64_t *sizes,
                uint64_t n, const Prescan &pre, int dir, int max_wgs, hipStream_t stream,
                hipStream_t up, uint32_t chunk, uint32_t flags, hipEvent_t ev_begin,
                hipEvent_t ev_end)
{
    if (s->recorded) {
        hipError_t e = hipEventSynchronize(s->done);   // the slot's previous kernel is done
        if (e != hipSuccess)
            return hip_fail(e);
    }
    int rc;
    if ((rc = reserve(s, pre.bound)) != KVCOPY_OK)
        return rc;
    const uint64_t n_chunks =
        build_worklist(src, dst, sizes, n, !(flags & KVCOPY_F_NO_COALESCE), chunk, s->host);

    const ChunkRec *recs = s->host;   // mapped: device-readable at the host address
    const bool upload = (flags & KVCOPY_F_DESC_UPLOAD) ||
                        (!(flags & KVCOPY_F_DESC_MAPPED) && n_chunks > KVCOPY_MAPPED_MAX_CHUNKS);
    if (upload) {
        // The copy runs on the library's stream, so it can overlap work that
        // is still queued on the caller's stream; the caller's stream then
        // waits for it before the kernel.  The device twin is free: the
        // slot's previous kernel has completed (waited on above).
        hipError_t e;
        if (s->uploaded == nullptr &&
            (e = hipEventCreateWithFlags(&s->uploaded, hipEventDisableTiming)) != hipSuccess)
            return hip_fail(e);
        if ((e = hipMemcpyAsync(s->dev, s->host, (size_t)n_chunks * sizeof(ChunkRec),
                                hipMemcpyHostToDevice, up)) != hipSuccess)
            return hip_fail(e);
        if ((e = hipEventRecord(s->uploaded, up)) != hipSuccess)
            return hip_fail(e);
        if ((e = hipStreamWaitEvent(stream, s->uploaded, 0)) != hipSuccess)
            return hip_fail(e);
        recs = s->dev;
    }
    hipError_t e;
    if (ev_begin && (e = hipEventRecord(ev_begin, stream)) != hipSuccess)
        return hip_fail(e);
    if ((e = launch_copy(recs, (uint32_t)n_chunks, grid_for(n_chunks, max_wgs), dir, stream)) !=
        hipSuccess)
        return hip_fail(e);
    if (ev_end && (e = hipEventRecord(ev_end, stream)) != hipSuccess)
        return hip_fail(e);
    if (s->done == nullptr &&
        (e = hipEventCreateWithFlags(&s->done, hipEventDisableTiming)) != hipSuccess)
        return hip_fail(e);
    if ((e = hipEventRecord(s->done, stream)) != hipSuccess)
        return hip_fail(e);
    s->recorded = true;
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
        if (opts->flags & ~(KVCOPY_F_VALIDATE | KVCOPY_F_NO_COALESCE | KVCOPY_F_DESC_MAPPED |
                            KVCOPY_F_DESC_UPLOAD))
            return KVCOPY_EINVAL;
        if ((opts->flags & KVCOPY_F_DESC_MAPPED) && (opts->flags & KVCOPY_F_DESC_UPLOAD))
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
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return hip_fail(e);
    DeviceRing *ring = ring_for(device);
    hipStream_t up = nullptr;
    if ((rc = upload_stream(ring, &up)) != KVCOPY_OK)
        return rc;
    Slot *slot;
    while ((slot = acquire(ring)) == nullptr)
        std::this_thread::yield();
    rc = run_in_slot(slot, src_addrs, dst_addrs, sizes, n, pre, dir, max_wgs, stream, up, chunk,
                     flags, ev_begin, ev_end);
    release(ring, slot);
    return rc;
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
