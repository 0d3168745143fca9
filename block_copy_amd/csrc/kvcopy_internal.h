// kvcopy_internal.h -- pieces shared by the planner, the runtime and the
// copy kernel of libkvcopy.  Not part of the public ABI (include/kvcopy.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace kvc {

// One entry of the chunk worklist the kernel consumes: a piece of one merged
// range, at most chunk_bytes long (a multiple of 16 except for the last
// piece of a range, which may end in an 8-byte word).
struct ChunkRec {
    uint64_t src;
    uint64_t dst;
    uint32_t bytes;
    uint32_t reserved;
};
static_assert(sizeof(ChunkRec) == 24, "ChunkRec is 24 bytes");

// ---- planner (plan.cpp) ----------------------------------------------------

// Drops zero sizes and (if `merge`) merges list-consecutive ranges that are
// adjacent in both source and destination.  Checks 8-byte alignment and
// address wrap-around.  Output arrays need room for n entries and may alias
// the inputs.  Returns KVCOPY_OK, KVCOPY_EALIGN or KVCOPY_EINVAL.
int merge_ranges(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
                 bool merge, uint64_t *osrc, uint64_t *odst, uint64_t *osize, uint64_t *m_out,
                 uint64_t *total_out);

// KVCOPY_EOVERLAP if any two destination ranges overlap or a destination
// overlaps a source range, else KVCOPY_OK.  Zero-size entries are ignored.
// O(m log m).
int check_overlap(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t m);

// begin[i] = sum over j < i of ceil(size[j] / chunk); begin has m + 1 entries.
// Returns begin[m].
uint64_t chunk_prefix(const uint64_t *size, uint64_t m, uint32_t chunk, uint64_t *begin);

// Writes the worklist: range i's chunks go to out[begin[i] .. begin[i+1]).
void emit_chunks(const uint64_t *src, const uint64_t *dst, const uint64_t *size,
                 const uint64_t *begin, uint64_t m, uint32_t chunk, ChunkRec *out);

// Facts about a descriptor list gathered in one read-only pass.
struct Prescan {
    uint64_t nnz;    // descriptors with a non-zero size
    uint64_t total;  // sum of sizes
    uint64_t bound;  // upper bound on the chunk count after merging: nnz + total / chunk
};

// One pass over the three input arrays: 8-byte alignment of every address and
// size (KVCOPY_EALIGN), no range wrapping past 2^64 and no overflowing total
// (KVCOPY_EINVAL).  Fills *out on success.
int prescan(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
            uint32_t chunk, Prescan *out);

// The batch path's fused planner: one sequential pass that checks what
// prescan() checks (same error codes, same priority), drops zero sizes,
// merges list-consecutive adjacent ranges (if `merge`) and writes each closed
// range's chunks straight into out[0 .. cap).  *n_chunks receives the number
// of records the batch needs, which may exceed cap: then only the first cap
// were written, and the caller plans again with room for *n_chunks.  The
// records are exactly those emit_chunks() gives for merge_ranges()'s output.
// With `stream`, the records are written with non-temporal stores (for the
// pinned staging ring, which only the GPU reads): call finish_records()
// before anything that hands them to the GPU.
int build_checked(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
                  bool merge, uint32_t chunk, ChunkRec *out, uint64_t cap, uint64_t *n_chunks,
                  bool stream = false);

// Orders every record streamed so far before the caller's later stores (the
// kernel launch's queue packet among them).
void finish_records();

// Whether build_checked plans this list with its AVX2 path (runs of
// single-chunk, non-adjacent descriptors four at a time): the host has AVX2
// and the list's first 64 descriptors are mostly such runs.
bool planner_vector_path(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
                         bool merge, uint32_t chunk);

// build_checked without the checks' result and without a cap (room for
// Prescan::bound records); returns how many records it wrote.
uint64_t build_worklist(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
                        bool merge, uint32_t chunk, ChunkRec *out);

// KVCOPY_F_DST_ORDER without an upload: writes in[0..n) to out in order of
// destination region -- a stable counting sort of the records by
// (dst >> 26) & 15, so the records of one 64 MiB destination region (and of
// regions 1 GiB apart) are consecutive, in list order within the region.
constexpr uint32_t kDstRegionShift = 26;
constexpr uint32_t kDstBuckets = 16;
void order_by_dst(const ChunkRec *in, uint64_t n, ChunkRec *out);

// KVCOPY_F_DST_ORDER with KVCOPY_F_DESC_UPLOAD: grouping by 4 MiB region
// made on the GPU (order_kernel.hip), for any worklist length.  in[0..n)
// are the uploaded records in list order, out[0..n) receives them grouped
// by (dst >> kOrderShift) & (kOrderKeys - 1) in key order (no set order
// within a key);
// header is kOrderHeaderBytes of zeroed device memory (256 counters, then
// 256 cursors) that the two kernels use and leave dirty.  Two launches on
// `stream` (the library's upload stream); `start` (may be null) is bound to
// the first one's start.  n == 0 launches nothing.
constexpr uint32_t kOrderShift = 22;
constexpr uint32_t kOrderKeys = 256;
constexpr uint32_t kOrderThreads = 256;
constexpr uint32_t kOrderPerWG = 1024;   // records per workgroup (then grid-stride)
constexpr uint32_t kOrderMaxGrid = 1024;
constexpr uint64_t kOrderHeaderBytes = 2 * 256 * sizeof(uint32_t);
hipError_t launch_order(const ChunkRec *in, uint32_t n, ChunkRec *out, uint32_t *header,
                        hipStream_t stream, hipEvent_t start);

// True when KVCOPY_VALIDATE=1 in the environment; any value other than
// unset, "0" or "1" makes *bad true (strict parsing).
bool env_validate(bool *bad);

// Records `wgs` as the KVCOPY_WGS_AUTO cap of `dir` on `device`.
void set_tuned_wgs(int device, int dir, int wgs);

// Records e as this thread's last HIP error (kvcopy_last_hip_error) and
// returns KVCOPY_EHIP.
int hip_fail(hipError_t e);

// ---- kernel launch (kvcopy_kernel.hip) -------------------------------------

constexpr uint32_t kWavesPerWG = 4;
constexpr uint32_t kThreadsPerWG = 64 * kWavesPerWG;

// A worklist small enough to travel in the kernel arguments (3,080 bytes of
// kernel arguments; HIP allows 4 KiB): no staging region, no completion
// event, and no round trip over the host link before the first copy.
constexpr uint32_t kInlineRecs = 128;
struct InlineWork {
    uint32_t n_chunks;
    uint32_t reserved;
    ChunkRec rec[kInlineRecs];
};

// Launches the per-chunk loop over an inline worklist (w.n_chunks <= kInlineRecs);
// sc1_stores, start and stop as for launch_copy.
hipError_t launch_copy_inline(const InlineWork &w, uint32_t grid, int dir, bool sc1_stores,
                              hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// Launches the copy kernel for `dir` (one kernel symbol per direction, loop
// and store form, same result): `grid` workgroups; wavefront w of W copies
// the chunks [w*C/W, (w+1)*C/W), one chunk at a time or, if `pipelined`, as
// a stream of 4 KiB pieces with two 16 KiB passes in flight.  `sc1_stores`
// selects the per-chunk loop's sc1|nt store form (copy_chunk.h,
// kSc1StorePolicy) instead of nt alone; pace_on / pace_period (wall-clock
// ticks, period 0 = none) time-slice the per-chunk loop's issue.  Both are
// ignored by the pipelined loop.  recs must be device-readable (device
// memory or mapped host memory).  `start` and `stop` (either may be null)
// are bound to the kernel's own start and completion (hipExtLaunchKernel's
// events), which costs no separate marker on the stream.  Returns the
// launch status.
hipError_t launch_copy(const ChunkRec *recs, uint32_t n_chunks, uint32_t grid, int dir,
                       bool pipelined, bool sc1_stores, uint32_t pace_on, uint32_t pace_period,
                       hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// kvcopy_batch_pair: two worklists (ra[0..ca), rb[0..cb)) in one kernel;
// every wavefront alternates between its shares of the two lists in
// proportion to their chunk counts.  sc1_stores as for launch_copy (the
// pair's default is the sc1|nt form); start / stop as for launch_copy.
hipError_t launch_copy_pair(const ChunkRec *ra, uint32_t ca, const ChunkRec *rb, uint32_t cb,
                            uint32_t grid, bool sc1_stores, hipStream_t stream, hipEvent_t start,
                            hipEvent_t stop);

// KVCOPY_F_WG_PER_CHUNK: `grid` workgroups; workgroup g copies chunks g,
// g + grid, ..., its four wavefronts sharing each chunk.  sc1_stores, start
// and stop as for launch_copy.
hipError_t launch_copy_wg(const ChunkRec *recs, uint32_t n_chunks, uint32_t grid, int dir,
                          bool sc1_stores, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// KVCOPY_F_DYNAMIC: the per-chunk loop with chunks claimed at run time.
// claim points at two zeroed device counters (next chunk, wavefronts done);
// every wavefront claims `grain` chunks at a time with an atomic add, one
// batch ahead, and the last wavefront to finish resets both counters to zero.
hipError_t launch_copy_dynamic(const ChunkRec *recs, uint32_t n_chunks, uint32_t grid, int dir,
                               uint32_t *claim, uint32_t grain, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop);

// Largest grid of one launch: 2^22 workgroups of 256 work-items (HIP
// limits a launch to fewer than 2^32 work-items).  A capped grid still
// copies every chunk, since each wavefront's share is computed from gridDim.
// With at most 2^24 wavefronts claiming at most 64 chunks each, a dynamic
// loop's claim counter reaches at most KVCOPY_MAX_CHUNKS + 2^30 < 2^32 (one
// overshooting claim per wavefront), so the 32-bit counter never wraps.
constexpr uint32_t kMaxGrid = 1u << 22;
static_assert((uint64_t)kMaxGrid * kThreadsPerWG < (1ull << 32), "launch too large");
static_assert(KVCOPY_MAX_CHUNKS + (uint64_t)kMaxGrid * kWavesPerWG * 64 < (1ull << 32),
              "a dynamic loop's claim counter could wrap");

// Workgroups for a batch of n_chunks under max_wgs (KVCOPY_WGS_ALL or a
// positive cap; KVCOPY_WGS_AUTO must be resolved first): one wavefront per
// chunk at most, and at most kMaxGrid.
inline uint32_t grid_for(uint64_t n_chunks, int max_wgs)
{
    uint64_t g = (n_chunks + kWavesPerWG - 1) / kWavesPerWG;   // one wavefront per chunk
    if (max_wgs != 0 /* KVCOPY_WGS_ALL */ && (uint64_t)max_wgs < g)
        g = (uint64_t)max_wgs;
    return (uint32_t)(g < kMaxGrid ? g : kMaxGrid);
}

// Workgroups for the workgroup-per-chunk loop: one per chunk at most, and at
// most kMaxGrid (workgroups then stride over the chunks, so a capped grid
// still copies every chunk; c + grid stays below 2^32 for c < 2^31).
inline uint32_t grid_for_wg(uint64_t n_chunks, int max_wgs)
{
    uint64_t g = n_chunks;
    if (max_wgs != 0 /* KVCOPY_WGS_ALL */ && (uint64_t)max_wgs < g)
        g = (uint64_t)max_wgs;
    return (uint32_t)(g < kMaxGrid ? g : kMaxGrid);
}

// The default store form (copy_chunk.h): sc1 for D2H batches on grids of
// three or more workgroups, nt otherwise.  Measured on MI355X with 16,384 x
// 4 KiB, a lone D2H batch moves 12.9 / 25.6 / 50.1 / 56.2 GB/s at 1 / 2 / 4
// / 8 workgroups with sc1 stores and 26.4 / 52.5 / 55.1 / 54.6 with nt;
// beside an H2D batch on another stream the two forms tie at 1-2
// workgroups per stream (19.5-19.9 and 37.0-37.3 GB/s for both), and sc1
// wins from 4 up (65.2 against 55.4 at 4, 96.7 against 67.5 at 8).
constexpr uint32_t kSc1MinGrid = 3;
inline bool default_sc1(int dir, uint32_t grid)
{
    return dir == 1 /* KVCOPY_D2H */ && grid >= kSc1MinGrid;
}

// Largest grid of the dynamic loop.  Every claim is an atomic add on one
// device word: measured on MI355X, 65,536 chunks at the full grid (16,384
// workgroups, one chunk per claim) took 2.2 ms instead of 0.1 ms, the
// claims serialising at about 17 ns each; 128 workgroups keep the claims a
// small part of a call.
constexpr uint32_t kDynMaxGrid = 128;

// Chunks per claim: about four claims per wavefront, at most 64 (one record
// per lane), at least 1.
inline uint32_t claim_grain(uint64_t n_chunks, uint32_t grid)
{
    const uint64_t per = n_chunks / (4ull * grid * kWavesPerWG);
    return per < 1 ? 1u : per > 64 ? 64u : (uint32_t)per;
}

// The library's choice of copy loop when no loop flag forces one: the
// pipelined loop for D2D grids of at most 256 workgroups in which every
// wavefront has at least two chunks, else the per-chunk loop.  (On the host
// link the pipelined loop moves more bytes per workgroup at small grids but
// lengthens co-running kernels' worst steps several times over, and small
// grids are the setting chosen to protect them; there it is opt-in.)
inline bool pipeline_pays(int dir, uint32_t grid, uint64_t n_chunks)
{
    return dir == 2 /* KVCOPY_D2D */ && grid <= 256u && n_chunks >= 2ull * grid * kWavesPerWG;
}

// kvcopy_batch_pair: how many of the launch's nw wavefronts copy list a
// (the rest copy list b), in proportion to the chunk counts ca and cb,
// rounded to nearest, and at least one for each non-empty list.  nw >= 2
// whenever both lists are non-empty (a launch has at least 4 wavefronts).
inline uint32_t pair_split(uint64_t ca, uint64_t cb, uint32_t nw)
{
    if (ca == 0)
        return 0;
    if (cb == 0)
        return nw;
    const double share = (double)nw * (double)ca / ((double)ca + (double)cb);
    uint64_t wa = (uint64_t)(share + 0.5);
    if (wa < 1)
        wa = 1;
    if (wa > nw - 1u)
        wa = nw - 1u;
    return (uint32_t)wa;
}

// ---- device-resident batches (device_batch.hip) ---------------------------

uint64_t device_workspace_bytes(uint64_t max_n);

// Enqueues the plan kernel (one workgroup) and the copy kernel (`grid`
// workgroups) on `stream`.  status_out (device memory, may be null) also
// receives the workspace's status word.
hipError_t launch_device_batch(const uint64_t *src, const uint64_t *dst, const uint64_t *size,
                               const uint64_t *d_n, uint64_t max_n, uint32_t chunk, uint32_t grid,
                               void *workspace, uint64_t *status_out, hipStream_t stream);

// kvcopy_batch_device_noalloc: the device address of the library's own
// workspace array on `device` (which must be the current device), looked up
// on the first call per device.
hipError_t noalloc_workspace(int device, void **out);
uint64_t noalloc_workspace_bytes();

}  // namespace kvc
