// jobs.cpp -- paced submission of a batch in pieces, with completion
// backpressure (kvcopy_job_*).
//
// PegaFlow issue #408, "Follow-up", item 2: splitting a transfer into
// pieces only shortens the decode tail when the next piece is submitted
// after the previous one completed; the page places that progress in the
// transfer worker as an event-driven state machine (submit, record and query
// an event, yield while incomplete, advance), and its "Proposed direction"
// names the option chunk_descriptors.  A job is that state machine; the
// caller's worker drives it with kvcopy_job_poll.
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "kvcopy.h"
#include "kvcopy_internal.h"

struct kvcopy_job {
    std::vector<uint64_t> src, dst, size;
    uint64_t next = 0;          // first descriptor of the next piece
    uint64_t piece = 0;         // descriptors per piece
    int dir = 0, max_wgs = 0;
    hipStream_t stream = nullptr;
    hipEvent_t ev = nullptr;    // recorded after the piece in flight
    bool in_flight = false;
};

extern "C" int kvcopy_job_create(const uint64_t *src_addrs, const uint64_t *dst_addrs,
                                 const uint64_t *sizes, uint64_t n, int dir, int max_wgs,
                                 uint64_t piece_descs, hipStream_t stream, kvcopy_job_t **out)
{
    if (out == nullptr)
        return KVCOPY_EINVAL;
    *out = nullptr;
    if (dir != KVCOPY_H2D && dir != KVCOPY_D2H && dir != KVCOPY_D2D)
        return KVCOPY_EINVAL;
    if (max_wgs < KVCOPY_WGS_AUTO || n > KVCOPY_MAX_DESCS || (n > 0 && (!src_addrs || !dst_addrs || !sizes)))
        return KVCOPY_EINVAL;
    bool bad_env = false;
    const bool validate = kvc::env_validate(&bad_env);
    if (bad_env)
        return KVCOPY_EINVAL;
    kvc::Prescan pre;
    int rc = kvc::prescan(src_addrs, dst_addrs, sizes, n, KVCOPY_CHUNK_DEFAULT, &pre);
    if (rc != KVCOPY_OK)
        return rc;
    if (validate && (rc = kvc::check_overlap(src_addrs, dst_addrs, sizes, n)) != KVCOPY_OK)
        return rc;
    kvcopy_job_t *job = new (std::nothrow) kvcopy_job_t();
    if (job == nullptr)
        return KVCOPY_ENOMEM;
    try {
        job->src.assign(src_addrs, src_addrs + n);
        job->dst.assign(dst_addrs, dst_addrs + n);
        job->size.assign(sizes, sizes + n);
    } catch (...) {
        delete job;
        return KVCOPY_ENOMEM;
    }
    job->piece = piece_descs ? piece_descs : (n ? n : 1);
    job->dir = dir;
    job->max_wgs = max_wgs;
    job->stream = stream;
    *out = job;
    return KVCOPY_OK;
}

namespace {

// Submits the next piece; the event is recorded after its kernel.
int submit_next(kvcopy_job_t *job)
{
    const uint64_t n = job->src.size();
    const uint64_t k = job->next;
    const uint64_t m = n - k < job->piece ? n - k : job->piece;
    if (job->ev == nullptr) {
        const hipError_t e = hipEventCreateWithFlags(&job->ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            job->ev = nullptr;
            return kvc::hip_fail(e);
        }
    }
    int rc = kvcopy_batch(job->src.data() + k, job->dst.data() + k, job->size.data() + k, m,
                          job->dir, job->max_wgs, job->stream);
    if (rc != KVCOPY_OK)
        return rc;
    const hipError_t e = hipEventRecord(job->ev, job->stream);
    if (e != hipSuccess)
        return kvc::hip_fail(e);
    job->next = k + m;
    job->in_flight = true;
    return KVCOPY_OK;
}

}  // namespace

extern "C" int kvcopy_job_poll(kvcopy_job_t *job, int *done)
{
    if (job == nullptr || done == nullptr)
        return KVCOPY_EINVAL;
    *done = 0;
    if (job->in_flight) {
        const hipError_t e = hipEventQuery(job->ev);
        if (e == hipErrorNotReady)
            return KVCOPY_OK;
        if (e != hipSuccess)
            return kvc::hip_fail(e);
        job->in_flight = false;
    }
    if (job->next >= job->src.size()) {
        *done = 1;
        return KVCOPY_OK;
    }
    return submit_next(job);
}

extern "C" int kvcopy_job_wait(kvcopy_job_t *job)
{
    if (job == nullptr)
        return KVCOPY_EINVAL;
    for (;;) {
        int done = 0;
        int rc = kvcopy_job_poll(job, &done);
        if (rc != KVCOPY_OK || done)
            return rc;
        if (job->in_flight) {
            const hipError_t e = hipEventSynchronize(job->ev);
            if (e != hipSuccess)
                return kvc::hip_fail(e);
        }
    }
}

extern "C" void kvcopy_job_destroy(kvcopy_job_t *job)
{
    if (job == nullptr)
        return;
    if (job->ev)
        (void)hipEventDestroy(job->ev);
    delete job;
}
