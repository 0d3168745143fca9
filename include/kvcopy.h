/*
 * kvcopy.h -- C ABI of the batched descriptor copy for AMD Instinct MI355X (gfx950).
 *
 * One call moves a batch of n descriptors (src_addr, dst_addr, size): raw
 * device-visible addresses and byte counts of small, non-contiguous blocks
 * such as KV-cache pages or MoE expert bank rows.  Blocks move between
 * mapped pinned host memory and HBM (H2D, D2H) or within HBM (D2D).  The
 * whole batch costs one host planning pass and one kernel launch, instead of
 * one DMA memcpy per fragment; the planned worklist reaches the GPU through
 * library-owned pinned memory that the kernel reads in place, or, for a
 * batch of at most 128 chunks, in the kernel arguments.
 *
 * Sources (cited by page title and section):
 *   [PF]  PegaFlow issue #408, "Kernel transfer backend causes decode TPOT
 *         tail spikes under concurrent KV transfers".
 *   [VL]  vLLM PR #42212 report, "[Perf] Triton fast path for small CPU->GPU
 *         swap_blocks_batch in the offloading connector".
 *   [FT]  FreeToken issue #751, "[Perf] Offloaded decode: gather missed
 *         experts with a few TMA bulk-copy CTAs (cp.async.bulk, .shared::cta)
 *         instead of 48 x 1024 LDG threads".
 *
 * Conventions shared by every entry point:
 *   - Every function returns KVCOPY_OK (0) or a negative KVCOPY_E* code.
 *     Nothing aborts, throws or prints.
 *   - Invalid arguments are rejected before anything is enqueued.
 *   - Descriptor arrays are three parallel host arrays of n uint64 values,
 *     the layout of the three int64 address/size tensors in [VL] "key source
 *     snippet".  The caller owns them; no entry point keeps a pointer to them
 *     after it returns.
 *   - Addresses must be device-visible: device memory, or mapped pinned host
 *     memory whose device address equals its host address (see
 *     kvcopy_host_alloc_mapped).  Every address and every size must be a
 *     multiple of 8 bytes.  A size that is not a multiple of 8 is rejected,
 *     never truncated.
 *   - Destinations must not overlap each other or any source (memcpy, not
 *     memmove, semantics).  This is checked only in validate mode; otherwise
 *     such input is undefined.  Sources may overlap each other.
 *   - The result of a batch is exactly that of one memcpy per descriptor;
 *     under the rule above it does not depend on descriptor order, on the
 *     chunk size, on max_wgs or on dir.
 */
#ifndef KVCOPY_H
#define KVCOPY_H

#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t, hipEvent_t only */

#ifdef __cplusplus
extern "C" {
#endif

/* Direction hint.  It selects tuning only (which side is host-mapped); the
 * bytes moved never depend on it.  [PF] "Test setup": H2D and D2H are
 * submitted concurrently on separate streams. */
enum {
    KVCOPY_H2D = 0, /* src in mapped pinned host memory, dst in device memory */
    KVCOPY_D2H = 1, /* src in device memory, dst in mapped pinned host memory */
    KVCOPY_D2D = 2  /* both in device memory */
};

/* Status codes. */
enum {
    KVCOPY_OK = 0,
    KVCOPY_EINVAL = -1,   /* null pointer with n > 0, bad dir, max_wgs < -1, bad option, n too large */
    KVCOPY_EALIGN = -2,   /* an address or size is not a multiple of 8 bytes */
    KVCOPY_EOVERLAP = -3, /* validate mode: destinations overlap each other or a source */
    KVCOPY_ENOMEM = -4,   /* host or device allocation failed */
    KVCOPY_EHIP = -5      /* a HIP call failed; kvcopy_last_hip_error() has its code */
};

/* max_wgs == KVCOPY_WGS_ALL: one wavefront per chunk (the full grid).  The
 * "current full grid" of [PF] "Relevant implementation" launched one block
 * per descriptor.
 * max_wgs == KVCOPY_WGS_AUTO: the device's tuned cap for `dir` when
 * kvcopy_autotune has run on this device, else a fixed default measured on
 * MI355X: 128 for H2D and D2H (the best cap with both directions running
 * together; either direction alone already fills the host link with 8),
 * the full grid for D2D.  [PF] "Proposed direction": the cap should come
 * from a device-aware profile, not a universal constant. */
#define KVCOPY_WGS_ALL 0
#define KVCOPY_WGS_AUTO (-1)

/* Default chunk size: [FT] "What we changed" cuts the call's rows into
 * chunks of up to 16 KiB, each inside one row. */
#define KVCOPY_CHUNK_DEFAULT 16384u
#define KVCOPY_CHUNK_MAX (1u << 20)

/* Largest accepted n and largest number of chunks in one call. */
#define KVCOPY_MAX_DESCS ((uint64_t)1 << 31)
#define KVCOPY_MAX_CHUNKS ((uint64_t)1 << 31)

/* Option flags for kvcopy_batch_ex.  By default the kernel reads the
 * worklist in place from the library's pinned staging ring (it crosses the
 * host link once, as part of the kernel's own loads); KVCOPY_F_DESC_UPLOAD
 * first copies it into device memory with hipMemcpyAsync on a stream of the
 * library's own (one per device, default priority, created on first use),
 * and `stream` waits for that copy (and, with KVCOPY_F_DST_ORDER, the two
 * order kernels that follow it there) before the kernel: in a train of
 * calls they overlap the previous call's kernel.  The library's device copy
 * of its staging ring (two halves, the second for ordered worklists) is
 * allocated on the first such call. */
#define KVCOPY_F_VALIDATE 0x1u    /* check the overlap rule (O(n log n)); also on when KVCOPY_VALIDATE=1 */
#define KVCOPY_F_NO_COALESCE 0x2u /* skip merging of adjacent ranges (for measurement only) */
#define KVCOPY_F_DESC_UPLOAD 0x8u /* upload the worklist to device memory before the kernel */
/* Copy loop.  Two loops give the same bytes: the per-chunk loop (a
 * wavefront has one chunk's loads in flight) and the pipelined loop (a
 * wavefront streams its chunks as 4 KiB pieces with two 16 KiB passes in
 * flight).  By default D2D calls use the pipelined loop when the grid has at
 * most 256 workgroups and every wavefront at least two chunks, and all other
 * calls the per-chunk loop.  Measured on MI355X: with 1-4 workgroups the
 * pipelined loop moves 35-40% more bytes per workgroup over the host link,
 * but it lengthens a co-running decode loop's worst steps several times over
 * (small grids being the setting chosen to protect such work), and with both
 * host-link directions at 16+ workgroups each it cuts the pair's rate by a
 * third; so on the host link it is opt-in.  These flags force one loop
 * (setting more than one loop flag, KVCOPY_F_DYNAMIC and
 * KVCOPY_F_WG_PER_CHUNK below included, is KVCOPY_EINVAL). */
#define KVCOPY_F_PIPELINE 0x10u
#define KVCOPY_F_PER_CHUNK 0x20u
/* The per-chunk loop with chunks claimed at run time instead of an equal
 * contiguous share per wavefront: a wavefront claims a batch of chunks
 * (about a quarter of its fair share, at most 64) with an atomic add on a
 * counter in device memory, one batch ahead, so faster wavefronts take more
 * chunks.  The library owns the counters (allocated and zeroed on first use,
 * reset by each kernel's last wavefront).  Every claim hits one counter, so
 * this loop runs at most 128 workgroups whatever max_wgs allows (measured
 * on MI355X: 65,536 chunks at the full grid took 2.2 ms, the claims
 * serialising).  Exclusive with the two flags above. */
#define KVCOPY_F_DYNAMIC 0x40u
/* Store form of the per-chunk loop.  Two forms give the same bytes: the
 * nontemporal hint alone ("nt"), and nt with the sc1 scope bit ("sc1", a
 * device-scope store on the gfx940 family).  By default D2H batches use sc1
 * (nt on grids of one or two workgroups, where a lone D2H batch moves twice
 * as much with nt: 26.4 against 12.9 GB/s at one workgroup) and H2D and D2D
 * batches nt.  Measured on MI355X with 16,384 x 4 KiB each
 * way on two streams: 94.2-94.6 GB/s with the D2H kernel's stores in the
 * sc1 form, 87.9-88.4 with nt, whatever the H2D kernel's form; a lone D2H
 * batch 56.7 against 52.7 GB/s.  These flags force one form, for any
 * direction; they select the per-chunk loop unless KVCOPY_F_WG_PER_CHUNK
 * is given (KVCOPY_F_PIPELINE or KVCOPY_F_DYNAMIC with either is
 * KVCOPY_EINVAL, and so are both).
 * kvcopy_batch_pair takes KVCOPY_F_STORE_NT (its default is sc1). */
#define KVCOPY_F_STORE_SC1 0x80u
#define KVCOPY_F_STORE_NT 0x100u
/* Destination order: the worklist handed to the kernel is ordered by
 * destination region instead of list order, so that the chunks in flight at
 * any moment write a narrow band of memory.  Results do not depend on it.
 * Meant for D2D gathers of many random blocks.
 *   - With KVCOPY_F_DESC_UPLOAD the worklist is uploaded in list order and
 *     grouped on the GPU by 4 MiB region ((dst >> 22) mod 256; no set order
 *     within a region) by two small kernels that follow the upload on the
 *     library's stream, outside kernel_begin / kernel_end, so in a train of
 *     calls they run while the previous call's copy does.  Measured on
 *     MI355X with KVCOPY_F_WG_PER_CHUNK (below), D2D calls of 65,536 random
 *     4 KiB blocks between two 1 GiB pools: 95.8-96.0 us per copy kernel
 *     with sc1 stores (70% of 8 TB/s of HBM traffic; 93.1 on a list sorted
 *     by destination, 103.5 in list order), and back to back from C 96.2-
 *     96.7 us per call, the GPU's pace (60-65 us of host time per call).
 *     An isolated call takes longer than without the flags (about 190
 *     against 137 us from call to completion): the upload and the grouping
 *     come before the copy.
 *   - Otherwise the host groups the records by 64 MiB region
 *     ((dst >> 26) mod 16; list order within a region), a counting sort
 *     that costs about 60 us of host time per 65,536 records.  With the
 *     per-chunk loop, reading the records in place, the kernel gains 2-5%
 *     (101.6-104.8 against 107.0-107.6 us for the calls above). */
#define KVCOPY_F_DST_ORDER 0x200u
/* Tail-bounded policy ([PF] "Proposed direction": a tail-bounded policy
 * beside the throughput-oriented one, for transfers that share the GPU with
 * latency-sensitive kernels).  A preset of the options above: the sc1 store
 * form (unless KVCOPY_F_STORE_NT is given), a 2 us issue window in every
 * 20 us (unless duty_on_ns / duty_period_ns are given), and at most 4
 * workgroups per call (max_wgs above 4, KVCOPY_WGS_ALL and KVCOPY_WGS_AUTO
 * become 4).  It moves about 3.3 GB/s of 4 KiB blocks per call in flight.
 * Measured on MI355X with a batch-1 decode loop of 36 bf16 GEMVs (0.38 ms
 * per step) beside an H2D + D2H burst of 16,384 x 4 KiB each way every
 * 50 ms on two streams: decode step p99 +4.9% and worst step 0.43 ms
 * (0.41 ms with no transfer) at 2.61 GiB/s sustained, where the default
 * (128 workgroups per stream) gives p99 +2% but a worst step near 2 ms.
 * With KVCOPY_F_PIPELINE, KVCOPY_F_DYNAMIC or KVCOPY_F_WG_PER_CHUNK:
 * KVCOPY_EINVAL. */
#define KVCOPY_F_TAIL_BOUNDED 0x400u
/* One workgroup per chunk: the four wavefronts of a workgroup share each
 * chunk (thread t moves the 16-byte words at t*16 + k*4 KiB), and workgroup
 * g of G copies chunks g, g + G, g + 2G, ... .  The grid is max_wgs
 * workgroups, or one per chunk with KVCOPY_WGS_ALL (at most 2^22).  Each
 * workgroup reads its own chunk's record before its first data access, so
 * the worklist belongs in device memory: combine with KVCOPY_F_DESC_UPLOAD
 * (read in place from pinned host memory it ran at half the speed).  With
 * a worklist in destination order (KVCOPY_F_DST_ORDER, or a caller's list
 * sorted by destination) the workgroups that the dispatcher starts together
 * read and write whole blocks of a narrow band of memory: measured on
 * MI355X for D2D calls of 65,536 random 4 KiB blocks between two 1 GiB pools,
 * cycling over 8 distinct batches, with the records in device memory and
 * sc1 stores, 92.3-92.6 us per kernel with KVCOPY_F_DST_ORDER (5.8 TB/s of
 * HBM traffic, 73% of 8 TB/s) and 93.1 us on a list sorted by destination,
 * against 98.0 us for one wavefront per chunk on the sorted list, and 103.4
 * against 107.6 us in list order.  Takes the store forms above (default as
 * for the per-chunk loop); with another loop flag, pacing or
 * KVCOPY_F_TAIL_BOUNDED: KVCOPY_EINVAL. */
#define KVCOPY_F_WG_PER_CHUNK 0x800u

/*
 * kvcopy_coalesce -- merge list-consecutive adjacent ranges.
 *
 * [PF] "Relevant implementation": the memcpy backend merges adjacent ranges
 * and submits one copy per merged range.  Rule: one pass in list order, no
 * sort; zero-size descriptors are dropped; a descriptor joins the range
 * built so far when it starts where that range ends in BOTH source and
 * destination.  Host-only: no GPU work, no allocation.
 *
 * in:  src, dst, sizes -- n entries each (may be NULL when n == 0).
 * out: out_src, out_dst, out_sizes -- room for n entries; they may be the
 *      same arrays as the inputs (in-place).  *out_n receives the count m <= n.
 * errors: KVCOPY_EINVAL for a NULL array with n > 0 or a NULL out_n.
 *         No alignment check is made here.
 */
int kvcopy_coalesce(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes, uint64_t n,
                    uint64_t *out_src, uint64_t *out_dst, uint64_t *out_sizes, uint64_t *out_n);

/*
 * kvcopy_plan -- validate, coalesce and chunk a batch (host-only).
 *
 * [FT] "What we changed": the call's total bytes are cut into chunks of at
 * most chunk_bytes that never cross a range.  Merged range i of size s_i
 * owns c_i = ceil(s_i / chunk_bytes) chunks, numbered from chunk_begin[i] =
 * sum of c_j over j < i (an exclusive prefix sum); chunk k of range i covers
 * bytes [(k - chunk_begin[i]) * chunk_bytes, min(... + chunk_bytes, s_i)).
 *
 * chunk_bytes: 0 = KVCOPY_CHUNK_DEFAULT; else a multiple of 16, at most
 *              KVCOPY_CHUNK_MAX (else KVCOPY_EINVAL).
 * out: filled on success; the plan owns its arrays (release with
 *      kvcopy_plan_free).  src/dst/size have n_merged entries, chunk_begin
 *      n_merged + 1.
 * errors: KVCOPY_EINVAL, KVCOPY_EALIGN, KVCOPY_EOVERLAP (validate mode:
 *         KVCOPY_VALIDATE=1 in the environment), KVCOPY_ENOMEM.
 */
typedef struct {
    uint64_t n_in;        /* descriptors given */
    uint64_t n_merged;    /* ranges after dropping zero sizes and merging */
    uint64_t n_chunks;    /* chunk_begin[n_merged] */
    uint64_t total_bytes; /* sum of sizes */
    uint32_t chunk_bytes;
    uint32_t reserved;
    const uint64_t *src, *dst, *size; /* n_merged entries each */
    const uint64_t *chunk_begin;      /* n_merged + 1 entries */
} kvcopy_plan_t;

int kvcopy_plan(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes, uint64_t n,
                uint32_t chunk_bytes, kvcopy_plan_t *out);
void kvcopy_plan_free(kvcopy_plan_t *plan);

/*
 * kvcopy_batch -- enqueue the whole batch on `stream`; no host sync.
 *
 * [PF] "Summary": one descriptor upload and one copy-kernel launch replace
 * many directional memcpy submissions; "Follow-up", item 2: the transfer
 * contract is enqueue-only.  [VL] "key source snippet": the descriptor
 * arrays go to the GPU asynchronously from pinned buffers, then one
 * persistent copy kernel runs.
 *
 * The library plans the batch (coalesce, chunk), writes the chunk worklist
 * into its own pinned staging ring, and launches one kernel of
 * min(max_wgs, needed) workgroups of 4 wavefronts on `stream`.  Each
 * wavefront takes an equal contiguous share of the chunks and moves them
 * with 16-byte loads and nontemporal 16-byte stores (a D2H batch's stores
 * also carry the sc1 scope bit, which is faster over the host link; the
 * bytes moved are the same; see KVCOPY_F_STORE_SC1).  The staging region is
 * recycled once an event recorded after the kernel has completed; the call
 * waits on the host only if the whole ring is still in use.  A batch of at
 * most 128 chunks instead passes its worklist in the kernel arguments (no
 * staging region, no event).  Calls on one
 * device are serialised on the host while they plan (microseconds).  The
 * call is not capturable into a HIP graph: the worklist is planned on the
 * host at call time.
 *
 * src_addrs, dst_addrs, sizes: n entries (host arrays; may be NULL if n == 0).
 * n:       0 is a valid empty call (returns KVCOPY_OK, enqueues nothing).
 * dir:     KVCOPY_H2D / KVCOPY_D2H / KVCOPY_D2D (tuning only).
 * max_wgs: workgroup cap ([PF] "Follow-up", item 1: a bounded grid; "Proposed
 *          direction": max_grid_blocks).  KVCOPY_WGS_ALL (0) = one wavefront
 *          per chunk; KVCOPY_WGS_AUTO (-1) = the device's tuned or default
 *          cap.  Below -1 = KVCOPY_EINVAL.  Measured on MI355X, two copy
 *          kernels running at once on two streams overlap only while each
 *          stays within about 256 workgroups (1,024 wavefronts); past that
 *          they run as if one after the other.
 * stream:  HIP stream (NULL = the null stream) of the calling thread's
 *          current device: the staging ring, the completion events and the
 *          kernel all belong to that device.
 * Ownership: the descriptor arrays may be reused as soon as the call
 *          returns.  The payload memory must stay valid, and unwritten by
 *          others, until the stream has passed the copy.
 * Threads: calls from several threads on several streams are safe.
 * errors:  KVCOPY_EINVAL, KVCOPY_EALIGN, KVCOPY_EOVERLAP (validate mode),
 *          KVCOPY_ENOMEM, KVCOPY_EHIP.  On KVCOPY_EHIP the stream may hold
 *          part of the work.
 */
int kvcopy_batch(const uint64_t *src_addrs, const uint64_t *dst_addrs, const uint64_t *sizes,
                 uint64_t n, int dir, int max_wgs, hipStream_t stream);

/* Options for kvcopy_batch_ex.  Zero-initialise, then set struct_size.
 * struct_size may also be KVCOPY_OPTS_V1_SIZE (the layout without the
 * duty-cycle fields, which then count as zero). */
typedef struct {
    uint32_t struct_size;   /* sizeof(kvcopy_opts_t) or KVCOPY_OPTS_V1_SIZE */
    uint32_t chunk_bytes;   /* 0 = default; else a multiple of 16, <= KVCOPY_CHUNK_MAX */
    uint32_t flags;         /* KVCOPY_F_* */
    uint32_t reserved;
    hipEvent_t kernel_begin; /* if non-NULL: bound to the copy kernel's start (hipExtLaunchKernel;
                              * not the upload or the order kernels before it) */
    hipEvent_t kernel_end;   /* if non-NULL: bound to the copy kernel's completion */
    /* Time-sliced issue ([PF] "Proposed direction": a tail-bounded policy
     * that trades transfer speed for co-running kernels' latency).  When
     * duty_period_ns is non-zero, every wavefront starts a chunk only in the
     * first duty_on_ns of each duty_period_ns of the device's wall clock
     * (hipDeviceAttributeWallClockRate), so all copy kernels issue in the
     * same windows and leave the host link idle in between.  Requires
     * 1,000 <= duty_on_ns <= duty_period_ns <= 10,000,000 (else
     * KVCOPY_EINVAL); on == period means no pacing.  Applies to the
     * per-chunk loop (with KVCOPY_F_PIPELINE, KVCOPY_F_DYNAMIC or
     * KVCOPY_F_WG_PER_CHUNK: KVCOPY_EINVAL).  A chunk started at the end of a window still
     * completes after it, so the link carries traffic for somewhat longer
     * than duty_on_ns per period. */
    uint32_t duty_on_ns;
    uint32_t duty_period_ns;
} kvcopy_opts_t;
#define KVCOPY_OPTS_V1_SIZE 32u

/*
 * kvcopy_batch_ex -- kvcopy_batch with options (chunk size, flags, and
 * events bound to the copy kernel's own start and end, for timing: their
 * elapsed time is the kernel's execution alone).  Events must be created
 * with timing enabled.  opts may be NULL
 * (= kvcopy_batch).  Errors as kvcopy_batch, plus KVCOPY_EINVAL for a bad
 * struct_size, chunk_bytes or unknown flag.
 */
int kvcopy_batch_ex(const uint64_t *src_addrs, const uint64_t *dst_addrs, const uint64_t *sizes,
                    uint64_t n, int dir, int max_wgs, hipStream_t stream,
                    const kvcopy_opts_t *opts);

/*
 * kvcopy_batch_pair -- two descriptor lists in one kernel launch on `stream`.
 *
 * [PF] "Test setup": KV offload traffic arrives as H2D and D2H bursts at the
 * same time.  When both lists are at hand, this call moves them with one
 * kernel whose wavefronts are split between the lists in proportion to
 * their chunk counts, with every workgroup holding wavefronts of both, so
 * every CU in use carries both directions and both directions of the host
 * link stay busy together until the end.  Measured on MI355X with 16,384 x
 * 4 KiB each way: 98-99 GB/s, where the same bursts as two kernels on two
 * streams reach 93-94 GB/s (and less when the two caps differ: the
 * direction with fewer requests in flight loses its share of the link).
 * The bytes moved are exactly those of kvcopy_batch(a) followed by
 * kvcopy_batch(b) on `stream`.
 *
 * Each list is validated, coalesced and chunked (16 KiB) as by kvcopy_batch;
 * the overlap rule spans both lists (no destination may overlap another
 * destination or any source of either list; checked in validate mode).
 * The kernel reads and writes through the addresses as given, so either
 * list may hold any direction; the usual use is H2D in one and D2H in the
 * other.  n_a or n_b may be 0 (both 0: KVCOPY_OK, nothing enqueued).  By
 * default the kernel's stores carry the sc1 scope bit as well as the
 * nontemporal hint (as kvcopy_batch's D2H kernel does); KVCOPY_F_STORE_NT
 * selects the nontemporal hint alone.
 * max_wgs as for kvcopy_batch, except that KVCOPY_WGS_AUTO is 64
 * workgroups, the steadiest cap measured for the burst above (98.4 GB/s;
 * 96-160 workgroups reach 99.1-99.5 at the median with occasional slow
 * windows; the full grid 84).
 * flags: KVCOPY_F_VALIDATE, KVCOPY_F_NO_COALESCE and KVCOPY_F_STORE_NT, as
 * for kvcopy_batch_ex; any other bit is KVCOPY_EINVAL.  Ownership, threads and
 * errors as for kvcopy_batch; an error in either list enqueues nothing.
 */
int kvcopy_batch_pair(const uint64_t *src_a, const uint64_t *dst_a, const uint64_t *sizes_a,
                      uint64_t n_a, const uint64_t *src_b, const uint64_t *dst_b,
                      const uint64_t *sizes_b, uint64_t n_b, int max_wgs, uint32_t flags,
                      hipStream_t stream);

/* Static text for a status code ("unknown status" for others). */
const char *kvcopy_strerror(int code);

/* The hipError_t of this thread's last failed HIP call (0 if none). */
int kvcopy_last_hip_error(void);

/*
 * kvcopy_host_alloc_mapped -- pinned host memory that the GPU can address
 * at the same virtual address ([PF] "Test setup": the host payload is mapped
 * pinned memory).  bytes > 0; *out receives the pointer.
 * errors: KVCOPY_EINVAL (bytes == 0 or out NULL), KVCOPY_ENOMEM, KVCOPY_EHIP
 * (also if the device address differs from the host address).
 */
int kvcopy_host_alloc_mapped(uint64_t bytes, void **out);

/* Release memory from kvcopy_host_alloc_mapped.  NULL is a no-op. */
int kvcopy_host_free(void *p);

/*
 * Paced submission with completion backpressure.
 *
 * [PF] "Follow-up", item 2, and "Proposed direction": splitting a transfer
 * into pieces helps co-running decode only if each piece is submitted after
 * the previous one has completed; enqueueing all pieces at once does not,
 * and a fixed sleep adds nothing.  The progress belongs in the caller's
 * transfer worker as an event-driven state machine, which a job is: it
 * holds a batch split into pieces of at most `piece_descs` descriptors and
 * submits piece k+1 (as one kvcopy_batch on `stream`) only from a
 * kvcopy_job_poll call that finds piece k's kernel completed.  Nothing here
 * blocks except kvcopy_job_wait.
 *
 * kvcopy_job_create: copies the three arrays (the caller may reuse them at
 *   once); submits nothing.  piece_descs == 0 means one piece (the whole
 *   batch).  Validation as kvcopy_batch (the whole list is checked here, so
 *   a piece never fails on its arguments later).
 *   errors: KVCOPY_EINVAL (also out == NULL), KVCOPY_EALIGN, KVCOPY_EOVERLAP
 *   (validate mode), KVCOPY_ENOMEM.
 * kvcopy_job_poll: if no piece is in flight or the one in flight has
 *   completed, submits the next piece; *done = 1 once every piece has
 *   completed (then further polls do nothing).  Never waits.
 *   errors: KVCOPY_EINVAL (NULL job or done), as kvcopy_batch for a submit.
 * kvcopy_job_wait: polls until done, blocking on each piece's event.
 * kvcopy_job_destroy: frees the job (call it only once no piece is in
 *   flight, i.e. after done, or after a failed poll).  NULL is a no-op.
 * A job is used by one thread at a time.
 */
typedef struct kvcopy_job kvcopy_job_t;

int kvcopy_job_create(const uint64_t *src_addrs, const uint64_t *dst_addrs, const uint64_t *sizes,
                      uint64_t n, int dir, int max_wgs, uint64_t piece_descs, hipStream_t stream,
                      kvcopy_job_t **out);
int kvcopy_job_poll(kvcopy_job_t *job, int *done);
int kvcopy_job_wait(kvcopy_job_t *job);
void kvcopy_job_destroy(kvcopy_job_t *job);

/*
 * kvcopy_autotune -- a startup probe that picks the workgroup cap.
 *
 * [FT] "Proposal", question 1, suggests choosing the worker count from a
 * small startup probe and targeting bytes in flight rather than threads;
 * the vLLM PR #42212 report ("key source snippet", the tuned constants)
 * picks the smallest number of workers within a tolerance of peak
 * bandwidth.  This call probes the current device and keeps a tolerance,
 * but breaks ties the other way (below): it allocates its
 * own probe buffers (64 MiB of mapped pinned host memory and 64 MiB of
 * device memory per direction, freed before it returns), times 24 batches
 * of 16,384 shuffled 4 KiB blocks per direction at each cap of
 * KVCOPY_AUTOTUNE_CAPS, after four untimed ones (for H2D or D2H both
 * directions run together, H2D on s0 and D2H on s1, joined at every step
 * as in a KV offload burst; D2D runs on s0), in three sweeps over the caps
 * (ascending, descending, ascending), and rates each cap by its median
 * sweep.  It records as the device's KVCOPY_WGS_AUTO cap for `dir` (for H2D
 * or D2H: for both) the largest cap whose median is within 2% of the best
 * cap's.  Near-ties go to the larger grid: on MI355X, with two streams, 8
 * and 64 workgroups per stream rated within 0.5-1.1% of each other, but 8
 * later ran some 20-step windows of the burst 5-9% slower, 64 none.
 * Blocks until done (one to two seconds).
 * s0, s1: the streams the caller will copy on (the hardware queues they map
 *   to matter); NULL = streams created for the probe.
 * out_wgs (may be NULL): the chosen cap (0 = full grid).
 * out_rates (may be NULL): KVCOPY_AUTOTUNE_NCAPS doubles, bytes per second
 *   at each cap (median sweep), in the order of KVCOPY_AUTOTUNE_CAPS.
 * errors: KVCOPY_EINVAL (bad dir), KVCOPY_ENOMEM, KVCOPY_EHIP.
 */
#define KVCOPY_AUTOTUNE_NCAPS 10
#define KVCOPY_AUTOTUNE_CAPS {1, 2, 4, 8, 16, 32, 64, 128, 256, 0}
int kvcopy_autotune(int dir, hipStream_t s0, hipStream_t s1, int *out_wgs, double *out_rates);

/*
 * Device-resident batches (graph-capturable).
 *
 * [FT] "What we changed": the gather reads its miss count on the device, so
 * the launch has a fixed shape and a CUDA graph can capture it.  Here the
 * three descriptor arrays and the count live in device memory, written by
 * earlier GPU work; kvcopy_batch_device enqueues two kernels of fixed shape
 * on `stream` and does no host planning, allocation or synchronisation, so
 * the call can be captured in a HIP graph and replayed with new contents.
 *   1. one workgroup reads the count n (clamped to max_n), checks 8-byte
 *      alignment of every address and size, and writes into the workspace
 *      the exclusive prefix sum of the per-descriptor chunk counts
 *      ceil(size / chunk_bytes) (the chunk numbering of kvcopy_plan, but
 *      without coalescing);
 *   2. max_wgs workgroups copy the chunks, wavefront w of W taking chunks
 *      [w*C/W, (w+1)*C/W).
 * If any descriptor is misaligned, nothing is copied and the workspace's
 * first 64-bit word (its status) is KVCOPY_DEVICE_BAD_ALIGN; it is
 * KVCOPY_DEVICE_TOO_MANY_CHUNKS if the batch has 2^31 chunks or more, else
 * 0 once the plan kernel has run.  Destinations must not overlap each other or
 * a source (not checked on the device).
 *
 * d_src, d_dst, d_sizes: device arrays of max_n uint64 each (entries past
 *   the device count are not read).  d_n: device uint64, the count.
 * max_wgs: the copy kernel's workgroups; 0 selects 1024; KVCOPY_WGS_AUTO the
 *   device's tuned or default cap (1024 where that is the full grid).
 * chunk_bytes: 0 = KVCOPY_CHUNK_DEFAULT; else a multiple of 16, at most
 *   KVCOPY_CHUNK_MAX.
 * workspace: caller-owned device memory of kvcopy_device_workspace_bytes(max_n)
 *   bytes, 256-byte aligned; it must not be used by another call that may
 *   run at the same time.
 * errors (host side, nothing enqueued): KVCOPY_EINVAL (NULL pointer with
 *   max_n > 0, max_n > KVCOPY_MAX_DESCS, bad dir / max_wgs / chunk_bytes,
 *   misaligned workspace); KVCOPY_EHIP.  max_n == 0 is a no-op.
 */
#define KVCOPY_DEVICE_BAD_ALIGN 1
#define KVCOPY_DEVICE_TOO_MANY_CHUNKS 2

uint64_t kvcopy_device_workspace_bytes(uint64_t max_n);
int kvcopy_batch_device(const uint64_t *d_src, const uint64_t *d_dst, const uint64_t *d_sizes,
                        const uint64_t *d_n, uint64_t max_n, int dir, int max_wgs,
                        uint32_t chunk_bytes, void *workspace, hipStream_t stream);

/*
 * kvcopy_batch_device_noalloc -- kvcopy_batch_device with the library's own
 * workspace instead of a caller-allocated one.
 *
 * For callers that cannot allocate memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine): the
 * workspace is a file-scope device array of the library, of
 * kvcopy_device_workspace_bytes(KVCOPY_NOALLOC_MAX_N) bytes (1 MiB + 256 B),
 * which each GPU that the library runs on holds until the process ends.
 * Its device address is looked up on the first call on each device.
 *
 * Arguments and behaviour as for kvcopy_batch_device, except:
 *   max_n:    at most KVCOPY_NOALLOC_MAX_N (else KVCOPY_EINVAL, nothing
 *             enqueued).
 *   d_status: device uint64 (may be NULL) that receives the status word
 *             (0, KVCOPY_DEVICE_BAD_ALIGN or KVCOPY_DEVICE_TOO_MANY_CHUNKS)
 *             once the plan kernel has run; the workspace itself is not
 *             visible to the caller.
 * Every call on one GPU shares the one array: calls that may run at the
 * same time on one GPU (unordered streams) race and must not be made; calls
 * ordered on one stream are safe.  The array keeps the last call's
 * contents; each call rewrites everything it reads, so nothing needs
 * clearing.
 * errors: as kvcopy_batch_device; KVCOPY_EHIP also if the array's address
 *   cannot be looked up.
 */
#define KVCOPY_NOALLOC_MAX_N 131072u
int kvcopy_batch_device_noalloc(const uint64_t *d_src, const uint64_t *d_dst,
                                const uint64_t *d_sizes, const uint64_t *d_n, uint64_t max_n,
                                int dir, int max_wgs, uint32_t chunk_bytes, uint64_t *d_status,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVCOPY_H */
