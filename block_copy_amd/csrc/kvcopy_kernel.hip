// kvcopy_kernel.hip -- the persistent, workgroup-capped copy kernels (gfx950).
//
// Work unit: one chunk of the worklist (at most chunk_bytes, never crossing a
// range; FreeToken issue #751 "gather missed experts with a few TMA
// bulk-copy CTAs", section "What we changed", which deals such chunks to a
// few CTAs).  The grid is persistent, as in the vLLM PR #42212 report
// ("Triton fast path for small CPU->GPU swap_blocks_batch"), section "key
// source snippet", where a few programs loop over all jobs; here the job is a
// byte-bounded chunk instead of a whole descriptor, so a 1 MiB row is shared
// by many wavefronts while small rows are not left waiting.  The grid is
// capped by max_wgs (PegaFlow issue #408, "Follow-up", item 1: a bounded
// grid).  Each wavefront takes an equal contiguous share of the chunk list.
//
// Data path (CDNA4): each lane moves 16-byte vectors with
// buffer_load_dwordx4 / nontemporal buffer_store_dwordx4, lanes interleaved
// so that one wavefront instruction covers 1 KiB of contiguous bytes.
// Addresses only need 8-byte alignment: gfx950 serves 8-byte-aligned dwordx4
// accesses directly, so no head peeling or register shifting is needed when
// src and dst differ mod 16.  A range whose size is an odd multiple of 8
// ends in one 8-byte word.
//
// Two loops, same result:
//   - per-chunk: a wavefront issues the loads of one chunk (up to 16 KiB, 16
//     vectors per lane) before its first store, then moves to the next chunk;
//   - pipelined: a wavefront streams its chunks as 4 KiB pieces in passes of
//     16 KiB, the loads of the next pass in flight while the current one is
//     stored.  It keeps 16-32 KiB of reads outstanding per wavefront even
//     for 4 KiB descriptors, which pays when only a few workgroups run.
// The worklist records are fetched 64 at a time (one per lane) and one batch
// ahead in both loops.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kvcopy.h"
#include "kvcopy_internal.h"

namespace kvc {
namespace {

#include "copy_chunk.h"

// The persistent loop.  Wavefront w of W owns the contiguous chunk range
// [w*C/W, (w+1)*C/W): every wavefront gets the same number of chunks to
// within one, and every chunk is at most chunk_bytes, so the bytes are
// balanced.  The wavefront fetches its worklist records 64 at a time, one
// record per lane, with vector loads (the worklist may sit in pinned host
// memory: one round trip per 64 chunks), prefetching the next 64 while it
// copies the current ones, and hands each record to the whole wavefront with
// v_readlane.
struct Rec {
    uint64_t src, dst;
    uint32_t bytes;
};

__device__ __forceinline__ Rec load_rec(const ChunkRec *recs, uint32_t idx, bool valid)
{
    Rec r{0, 0, 0};
    if (valid) {
        const KVC_GLOBAL uint64_t *p =
            (const KVC_GLOBAL uint64_t *)reinterpret_cast<uintptr_t>(recs + idx);
        r.src = p[0];
        r.dst = p[1];
        r.bytes = (uint32_t)p[2];
    }
    return r;
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, uint32_t j)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, j);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), j);
    return ((uint64_t)hi << 32) | lo;
}

// Time-sliced issue (kvcopy_opts_t duty_on_ns / duty_period_ns): a
// wavefront starts a chunk only while the device's constant-rate wall clock
// (s_memrealtime, 100 MHz on MI355X) lies in the first `on` ticks of each
// `period`.  Every wavefront of every copy kernel reads the same clock, so
// all of them issue in the same windows and the host link has idle gaps
// between them.  period == 0: no pacing.  The host guarantees on >= 100
// ticks and period <= 1,000,000 ticks, and the poll below re-reads the clock
// every few ticks, so each wait ends within one period.
struct Pace {
    uint32_t on, period;   // wall-clock ticks
};

__device__ __forceinline__ void pace_wait(const Pace p)
{
    if (p.period == 0)
        return;
    for (;;) {
        const uint32_t t = (uint32_t)wall_clock64();
        if (t % p.period < p.on)
            return;
        __builtin_amdgcn_s_sleep(2);
    }
}

// Wavefront w of nw copies chunks [w*C/nw, (w+1)*C/nw) of the worklist,
// storing with cache policy SP.
template <int SP = kStorePolicy>
__device__ __forceinline__ void copy_share(const ChunkRec *__restrict__ recs, uint32_t n_chunks,
                                           uint32_t w, uint32_t nw, const Pace pace = Pace{0, 0})
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t lo = (uint32_t)((uint64_t)w * n_chunks / nw);
    const uint32_t hi = (uint32_t)((uint64_t)(w + 1) * n_chunks / nw);
    if (lo >= hi)
        return;
    Rec cur = load_rec(recs, lo + lane, lo + lane < hi);
    for (uint32_t base = lo; base < hi; base += 64u) {
        const uint32_t cnt = hi - base < 64u ? hi - base : 64u;
        const uint32_t nb = base + 64u;
        const Rec nxt = load_rec(recs, nb + lane, nb < hi && nb + lane < hi);   // prefetch
        for (uint32_t j = 0; j < cnt; ++j) {
            pace_wait(pace);
            copy_chunk<SP>(lane_u64(cur.src, j), lane_u64(cur.dst, j),
                           __builtin_amdgcn_readlane(cur.bytes, j), lane);
        }
        cur = nxt;
    }
}

template <int SP>
__device__ __forceinline__ void copy_worklist(const ChunkRec *__restrict__ recs, uint32_t n_chunks,
                                              const Pace pace)
{
    const uint32_t w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWG + (threadIdx.x >> 6));
    copy_share<SP>(recs, n_chunks, w, gridDim.x * kWavesPerWG, pace);
}

// ---- pipelined variant ------------------------------------------------------
//
// The loop above keeps one chunk's loads in flight per wavefront: with 4 KiB
// descriptors that is 4 KiB, and the wavefront waits a full memory round trip
// per chunk.  The pipelined loop instead cuts the wavefront's chunk list into
// a stream of pieces of at most 4 KiB (four 1 KiB rows) and moves them in
// passes of four pieces (16 KiB), two passes in flight: the loads of pass
// p+1 are issued before the stores of pass p, so a wavefront always has 16 to
// 32 KiB of reads outstanding whatever the descriptor size.  Pieces of one
// pass may come from different chunks.  A piece's 8-byte tail (a chunk that
// ends in an odd 8-byte word) rides in the same pass as one 8-byte access
// whose buffer range is empty when there is no tail, so the code has no
// per-piece branches and every wait is a counted vmcnt.
constexpr uint32_t kPieceBytes = 4096;
constexpr int kPiecesPerPass = 4;
constexpr int kRowsPerPiece = (int)(kPieceBytes / kRowBytes);
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

struct Piece {
    uint64_t src, dst;
    uint32_t len;   // 0: the stream is exhausted
};

__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// A buffer resource from wave-uniform values.  The values are uniform by
// construction, but the compiler may carry some of them through the loop in
// VGPRs; readfirstlane keeps the resource in SGPRs (without it the compiler
// wraps each access in a waterfall loop over the lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_u(uint64_t base, uint32_t bytes)
{
    return rsrc(uniform64(base), __builtin_amdgcn_readfirstlane(bytes));
}

// Worklist records through a buffer resource: lanes past the end of the
// wavefront's share read zeros, so the batch fetch needs no lane branches.
__device__ __forceinline__ Rec fetch_recs(const ChunkRec *recs, uint32_t first, uint32_t end,
                                          uint32_t lane)
{
    const uint32_t avail = first < end ? end - first : 0u;
    const uint32_t nrec = avail < 64u ? avail : 64u;
    const __amdgpu_buffer_rsrc_t r =
        rsrc_u(reinterpret_cast<uintptr_t>(recs + first), nrec * (uint32_t)sizeof(ChunkRec));
    const uint32_t o = lane * (uint32_t)sizeof(ChunkRec);
    const v2u s = __builtin_amdgcn_raw_buffer_load_b64(r, (int)o, 0, 0);
    const v2u d = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(o + 8), 0, 0);
    const uint32_t b = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(o + 16), 0, 0);
    return Rec{((uint64_t)s.y << 32) | s.x, ((uint64_t)d.y << 32) | d.x, b};
}

__device__ __forceinline__ uint32_t wave_incl_scan32(uint32_t v, uint32_t lane)
{
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(v, d, 64);
        v += lane >= d ? o : 0u;
    }
    return v;
}

// One batch of up to 64 chunks, one record per lane, seen as a list of
// pieces: lane j's chunk owns pieces [pstart_j, pend_j) of the batch.
struct PieceBatch {
    Rec rec;
    uint32_t pstart, pend;
    uint32_t total;   // pieces in the batch (wave-uniform)

    __device__ __forceinline__ void open(const Rec &r, uint32_t lane)
    {
        rec = r;
        const uint32_t pc = (r.bytes + kPieceBytes - 1u) / kPieceBytes;   // 0 past the share
        pend = wave_incl_scan32(pc, lane);
        pstart = pend - pc;
        total = __builtin_amdgcn_readlane(pend, 63);
    }
    // Piece q (wave-uniform); len 0 once q >= total.  No branches: the lane
    // that owns q is found with a ballot.
    __device__ __forceinline__ Piece at(uint32_t q) const
    {
        const uint64_t m = __ballot(q >= pstart && q < pend);
        const uint32_t j = m ? (uint32_t)__builtin_ctzll(m) : 0u;
        const uint32_t off = (q - __builtin_amdgcn_readlane(pstart, j)) * kPieceBytes;
        const uint32_t left = __builtin_amdgcn_readlane(rec.bytes, j) - off;
        const uint32_t len = left < kPieceBytes ? left : kPieceBytes;
        return Piece{lane_u64(rec.src, j) + off, lane_u64(rec.dst, j) + off, m ? len : 0u};
    }
};

template <int P>
__device__ __forceinline__ void load_pass(const Piece (&p)[P], v4u (&v)[P * kRowsPerPiece],
                                          v2u (&t)[P], uint32_t lane)
{
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const uint32_t body = p[k].len & ~15u;
        const __amdgpu_buffer_rsrc_t rs = rsrc_u(p[k].src, body);
#pragma unroll
        for (int r = 0; r < kRowsPerPiece; ++r)
            v[k * kRowsPerPiece + r] = __builtin_amdgcn_raw_buffer_load_b128(
                rs, (int)(lane * 16u + r * kRowBytes), 0, kLoadPolicy);
        const __amdgpu_buffer_rsrc_t rt = rsrc_u(p[k].src + body, p[k].len & 8u);
        t[k] = __builtin_amdgcn_raw_buffer_load_b64(rt, (int)(lane * 8u), 0, kLoadPolicy);
    }
}

template <int P>
__device__ __forceinline__ void store_pass(const Piece (&p)[P], const v4u (&v)[P * kRowsPerPiece],
                                           const v2u (&t)[P], uint32_t lane)
{
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const uint32_t body = p[k].len & ~15u;
        const __amdgpu_buffer_rsrc_t rd = rsrc_u(p[k].dst, body);
#pragma unroll
        for (int r = 0; r < kRowsPerPiece; ++r)
            __builtin_amdgcn_raw_buffer_store_b128(v[k * kRowsPerPiece + r], rd,
                                                   (int)(lane * 16u + r * kRowBytes), 0,
                                                   kStorePolicy);
        const __amdgpu_buffer_rsrc_t rt = rsrc_u(p[k].dst + body, p[k].len & 8u);
        __builtin_amdgcn_raw_buffer_store_b64(t[k], rt, (int)(lane * 8u), 0, kStorePolicy);
    }
}

__device__ __forceinline__ void copy_worklist_pipelined(const ChunkRec *__restrict__ recs,
                                                        uint32_t n_chunks)
{
    constexpr int P = kPiecesPerPass;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t nw = gridDim.x * kWavesPerWG;
    const uint32_t w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWG + (threadIdx.x >> 6));
    const uint32_t lo = (uint32_t)((uint64_t)w * n_chunks / nw);
    const uint32_t hi = (uint32_t)((uint64_t)(w + 1) * n_chunks / nw);
    if (lo >= hi)
        return;
    Rec nxt = fetch_recs(recs, lo, hi, lane);
    for (uint32_t base = lo; base < hi; base += 64u) {
        PieceBatch bt;
        bt.open(nxt, lane);
        nxt = fetch_recs(recs, base + 64u, hi, lane);   // prefetch the next batch
        Piece a[P], b[P];
        v4u va[P * kRowsPerPiece], vb[P * kRowsPerPiece];
        v2u ta[P], tb[P];
        uint32_t q = 0;
#pragma unroll
        for (int k = 0; k < P; ++k)
            a[k] = bt.at(q + k);
        q += P;
        load_pass(a, va, ta, lane);
        for (;;) {
#pragma unroll
            for (int k = 0; k < P; ++k)
                b[k] = bt.at(q + k);
            q += P;
            load_pass(b, vb, tb, lane);
            store_pass(a, va, ta, lane);
            if (q - P >= bt.total)
                break;
#pragma unroll
            for (int k = 0; k < P; ++k)
                a[k] = bt.at(q + k);
            q += P;
            load_pass(a, va, ta, lane);
            store_pass(b, vb, tb, lane);
            if (q - P >= bt.total)
                break;
        }
    }
}

// ---- dynamic claiming ---------------------------------------------------------
//
// The per-chunk loop over chunks claimed at run time: lane 0 adds `grain` to
// the call's claim counter (a device-memory atomic) and the wavefront copies
// the chunks [b, b + grain) it got, having already claimed and started
// fetching the records of its next batch.  The last wavefront to finish (the
// one whose increment of the done counter completes the grid) resets both
// counters to zero for the next call that uses them; every other wavefront
// has made its final claim before its own done increment, so no claim can
// follow the reset.
__device__ __forceinline__ uint32_t claim_batch(uint32_t *claim, uint32_t grain, uint32_t lane)
{
    uint32_t b = 0;
    if (lane == 0)
        b = atomicAdd(claim, grain);
    return __builtin_amdgcn_readfirstlane(b);
}

__device__ __forceinline__ void copy_worklist_dynamic(const ChunkRec *__restrict__ recs,
                                                      uint32_t n_chunks, uint32_t *claim,
                                                      uint32_t grain)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t nw = gridDim.x * kWavesPerWG;
    uint32_t b = claim_batch(claim, grain, lane);
    Rec cur = fetch_recs(recs, b, b < n_chunks ? (n_chunks - b < grain ? n_chunks : b + grain) : b,
                         lane);
    while (b < n_chunks) {
        const uint32_t cnt = n_chunks - b < grain ? n_chunks - b : grain;
        const uint32_t nb = claim_batch(claim, grain, lane);   // claim ahead
        const uint32_t ncnt = nb < n_chunks ? (n_chunks - nb < grain ? n_chunks - nb : grain) : 0u;
        const Rec nxt = fetch_recs(recs, nb, nb + ncnt, lane);
        for (uint32_t j = 0; j < cnt; ++j)
            copy_chunk(lane_u64(cur.src, j), lane_u64(cur.dst, j),
                       __builtin_amdgcn_readlane(cur.bytes, j), lane);
        cur = nxt;
        b = nb;
    }
    if (lane == 0) {
        if (atomicAdd(claim + 1, 1u) == nw - 1) {
            atomicExch(claim, 0u);
            atomicExch(claim + 1, 0u);
        }
    }
}

// ---- one workgroup per chunk ------------------------------------------------------
//
// Workgroup g of G copies chunks g, g + G, g + 2G, ...; its four wavefronts
// share each chunk: thread t moves the 16-byte words at t*16 + k*4 KiB, so a
// 4 KiB chunk is one load and one store per thread and a 16 KiB chunk four
// of each, all loads first.  The chunk's record is read by the workgroup
// itself (wave-uniform), just before its data: with the worklist in device
// memory and in destination order, the workgroups that the dispatcher
// starts together move whole blocks of a narrow band of memory.  Measured
// on MI355X with 65,536 random 4 KiB blocks between two 1 GiB pools (calls
// over 8 distinct batches, records in device memory): 95.6 us per kernel
// sorted by destination against 102.7 us with one wavefront per chunk.
constexpr uint32_t kWgRowBytes = kThreadsPerWG * 16u;   // one access per thread: 4 KiB
constexpr int kWgMaxRows = 4;                           // 16 KiB per pass

template <int R, int SP>
__device__ __forceinline__ void copy_wg_rows(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rd,
                                             uint32_t voff)
{
    v4u v[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(voff + j * kWgRowBytes), 0,
                                                     kLoadPolicy);
#pragma unroll
    for (int j = 0; j < R; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(v[j], rd, (int)(voff + j * kWgRowBytes), 0, SP);
}

// The whole workgroup copies one chunk.  src, dst and bytes are uniform.  As
// in copy_chunk, the buffer ranges end at the chunk's last whole 16-byte
// word, so the threads past the end of a short row need no masking, and an
// odd trailing 8-byte word is moved by thread 0.
template <int SP>
__device__ __forceinline__ void copy_chunk_wg(uint64_t src, uint64_t dst, uint32_t bytes)
{
    const uint32_t body = bytes & ~15u;
    const __amdgpu_buffer_rsrc_t rs = rsrc_u(src, body);
    const __amdgpu_buffer_rsrc_t rd = rsrc_u(dst, body);
    const uint32_t t16 = threadIdx.x * 16u;
    for (uint32_t off = 0; off < body; off += kWgRowBytes * kWgMaxRows) {
        const uint32_t left = body - off;
        switch (left >= kWgRowBytes * (kWgMaxRows - 1) + 1 ? kWgMaxRows
                                                           : (left + kWgRowBytes - 1) / kWgRowBytes) {
        case 1: copy_wg_rows<1, SP>(rs, rd, off + t16); break;
        case 2: copy_wg_rows<2, SP>(rs, rd, off + t16); break;
        case 3: copy_wg_rows<3, SP>(rs, rd, off + t16); break;
        default: copy_wg_rows<4, SP>(rs, rd, off + t16); break;
        }
    }
    if ((bytes & 8u) && threadIdx.x == 0) {   // a range that ends in an odd 8-byte word
        const uint64_t w = *reinterpret_cast<KVC_GLOBAL const uint64_t *>(src + body);
        __builtin_nontemporal_store(w, reinterpret_cast<KVC_GLOBAL uint64_t *>(dst + body));
    }
}

template <int SP>
__device__ __forceinline__ void copy_worklist_wg(const ChunkRec *__restrict__ recs,
                                                 uint32_t n_chunks)
{
    // c + gridDim.x cannot wrap: n_chunks <= 2^31 and gridDim.x <= 2^22
    for (uint32_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const KVC_GLOBAL uint64_t *p =
            (const KVC_GLOBAL uint64_t *)reinterpret_cast<uintptr_t>(recs + c);
        const uint64_t s = uniform64(p[0]), d = uniform64(p[1]);
        const uint32_t b = __builtin_amdgcn_readfirstlane((uint32_t)p[2]);
        copy_chunk_wg<SP>(s, d, b);
    }
}

// ---- two worklists in one launch -------------------------------------------------
//
// kvcopy_batch_pair: two worklists (typically an H2D burst and a D2H burst)
// in one kernel.  The launch's nw = 4G wavefronts are numbered slot-major,
// v = (wave in workgroup) * G + workgroup, and the first wa of them (wa
// chosen on the host in proportion to the chunk counts, pair_split) take
// list a, the rest list b, each list dealt out as in the per-chunk loop.
// With equal lists, waves 0-1 of every workgroup copy list a and waves 2-3
// list b, so every workgroup, and so every CU it runs on, carries both
// directions.  Measured on MI355X with 16,384 x 4 KiB each way at 64
// workgroups: 96.9 GB/s this way, 95.6 GB/s with each wavefront alternating
// between the lists, 82-85 GB/s with whole workgroups given to one list, and
// 65 GB/s with each wavefront copying its share of a and then of b.
template <int SP>
__device__ __forceinline__ void copy_pair(const ChunkRec *__restrict__ ra, uint32_t ca,
                                          const ChunkRec *__restrict__ rb, uint32_t cb,
                                          uint32_t wa)
{
    const uint32_t nw = gridDim.x * kWavesPerWG;
    const uint32_t v = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) * gridDim.x + blockIdx.x);
    if (v < wa)
        copy_share<SP>(ra, ca, v, wa);
    else
        copy_share<SP>(rb, cb, v - wa, nw - wa);
}

// ---- inline worklist ----------------------------------------------------------
//
// The per-chunk loop over a worklist passed by value in the kernel
// arguments: the records are read with scalar loads from the kernel-argument
// segment, so nothing crosses the host link before the first data load.
template <int SP>
__device__ __forceinline__ void copy_inline(const InlineWork &w)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t nw = gridDim.x * kWavesPerWG;
    const uint32_t wv = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWG + (threadIdx.x >> 6));
    const uint32_t n = w.n_chunks;
    const uint32_t lo = wv * n / nw, hi = (wv + 1) * n / nw;   // n <= 128: no overflow
    for (uint32_t j = lo; j < hi; ++j) {
        const uint32_t k = __builtin_amdgcn_readfirstlane(j);
        copy_chunk<SP>(w.rec[k].src, w.rec[k].dst, w.rec[k].bytes, lane);
    }
}

// One symbol per direction, loop and store form, so that profiles and
// counters separate them.  "_sc1" kernels store with kSc1StorePolicy, the
// others with kStorePolicy.
#define KVC_KERNEL(name, SP)                                                                       \
    __global__ __launch_bounds__(kThreadsPerWG) void name(const ChunkRec *__restrict__ recs,     \
                                                          uint32_t n_chunks, const Pace pace)    \
    {                                                                                              \
        copy_worklist<SP>(recs, n_chunks, pace);                                                   \
    }
KVC_KERNEL(kvcopy_h2d_kernel, kStorePolicy)
KVC_KERNEL(kvcopy_d2h_kernel, kStorePolicy)
KVC_KERNEL(kvcopy_d2d_kernel, kStorePolicy)
KVC_KERNEL(kvcopy_h2d_sc1_kernel, kSc1StorePolicy)
KVC_KERNEL(kvcopy_d2h_sc1_kernel, kSc1StorePolicy)
KVC_KERNEL(kvcopy_d2d_sc1_kernel, kSc1StorePolicy)
#undef KVC_KERNEL

#define KVC_PIPE_KERNEL(name)                                                                      \
    __global__ __launch_bounds__(kThreadsPerWG) void name(const ChunkRec *__restrict__ recs,     \
                                                          uint32_t n_chunks)                     \
    {                                                                                              \
        copy_worklist_pipelined(recs, n_chunks);                                                   \
    }
KVC_PIPE_KERNEL(kvcopy_h2d_pipe_kernel)
KVC_PIPE_KERNEL(kvcopy_d2h_pipe_kernel)
KVC_PIPE_KERNEL(kvcopy_d2d_pipe_kernel)
#undef KVC_PIPE_KERNEL

#define KVC_WG_KERNEL(name, SP)                                                                    \
    __global__ __launch_bounds__(kThreadsPerWG) void name(const ChunkRec *__restrict__ recs,     \
                                                          uint32_t n_chunks)                     \
    {                                                                                              \
        copy_worklist_wg<SP>(recs, n_chunks);                                                      \
    }
KVC_WG_KERNEL(kvcopy_h2d_wg_kernel, kStorePolicy)
KVC_WG_KERNEL(kvcopy_d2h_wg_kernel, kStorePolicy)
KVC_WG_KERNEL(kvcopy_d2d_wg_kernel, kStorePolicy)
KVC_WG_KERNEL(kvcopy_h2d_wg_sc1_kernel, kSc1StorePolicy)
KVC_WG_KERNEL(kvcopy_d2h_wg_sc1_kernel, kSc1StorePolicy)
KVC_WG_KERNEL(kvcopy_d2d_wg_sc1_kernel, kSc1StorePolicy)
#undef KVC_WG_KERNEL

#define KVC_PAIR_KERNEL(name, SP)                                                                  \
    __global__ __launch_bounds__(kThreadsPerWG) void name(                                         \
        const ChunkRec *__restrict__ ra, uint32_t ca, const ChunkRec *__restrict__ rb, uint32_t cb, \
        uint32_t wa)                                                                               \
    {                                                                                              \
        copy_pair<SP>(ra, ca, rb, cb, wa);                                                         \
    }
KVC_PAIR_KERNEL(kvcopy_pair_kernel, kSc1StorePolicy)
KVC_PAIR_KERNEL(kvcopy_pair_nt_kernel, kStorePolicy)
#undef KVC_PAIR_KERNEL

#define KVC_INLINE_KERNEL(name, SP)                                                                \
    __global__ __launch_bounds__(kThreadsPerWG) void name(const InlineWork w)                     \
    {                                                                                              \
        copy_inline<SP>(w);                                                                        \
    }
KVC_INLINE_KERNEL(kvcopy_h2d_inline_kernel, kStorePolicy)
KVC_INLINE_KERNEL(kvcopy_d2h_inline_kernel, kStorePolicy)
KVC_INLINE_KERNEL(kvcopy_d2d_inline_kernel, kStorePolicy)
KVC_INLINE_KERNEL(kvcopy_h2d_inline_sc1_kernel, kSc1StorePolicy)
KVC_INLINE_KERNEL(kvcopy_d2h_inline_sc1_kernel, kSc1StorePolicy)
KVC_INLINE_KERNEL(kvcopy_d2d_inline_sc1_kernel, kSc1StorePolicy)
#undef KVC_INLINE_KERNEL

#define KVC_DYN_KERNEL(name)                                                                       \
    __global__ __launch_bounds__(kThreadsPerWG) void name(const ChunkRec *__restrict__ recs,     \
                                                          uint32_t n_chunks, uint32_t *claim,    \
                                                          uint32_t grain)                        \
    {                                                                                              \
        copy_worklist_dynamic(recs, n_chunks, claim, grain);                                       \
    }
KVC_DYN_KERNEL(kvcopy_h2d_dyn_kernel)
KVC_DYN_KERNEL(kvcopy_d2h_dyn_kernel)
KVC_DYN_KERNEL(kvcopy_d2d_dyn_kernel)
#undef KVC_DYN_KERNEL

}  // namespace

hipError_t launch_copy(const ChunkRec *recs, uint32_t n_chunks, uint32_t grid, int dir,
                       bool pipelined, bool sc1_stores, uint32_t pace_on, uint32_t pace_period,
                       hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    static const void *const per_chunk[2][3] = {
        {reinterpret_cast<const void *>(&kvcopy_h2d_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2h_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2d_kernel)},
        {reinterpret_cast<const void *>(&kvcopy_h2d_sc1_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2h_sc1_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2d_sc1_kernel)}};
    static const void *const pipe[3] = {reinterpret_cast<const void *>(&kvcopy_h2d_pipe_kernel),
                                        reinterpret_cast<const void *>(&kvcopy_d2h_pipe_kernel),
                                        reinterpret_cast<const void *>(&kvcopy_d2d_pipe_kernel)};
    if (pipelined) {
        void *args[] = {(void *)&recs, (void *)&n_chunks};
        return hipExtLaunchKernel(pipe[dir], dim3(grid), dim3(kThreadsPerWG), args, 0, stream,
                                  start, stop, 0);
    }
    Pace pace{pace_on, pace_period};
    void *args[] = {(void *)&recs, (void *)&n_chunks, (void *)&pace};
    return hipExtLaunchKernel(per_chunk[sc1_stores ? 1 : 0][dir], dim3(grid), dim3(kThreadsPerWG),
                              args, 0, stream, start, stop, 0);
}

hipError_t launch_copy_wg(const ChunkRec *recs, uint32_t n_chunks, uint32_t grid, int dir,
                          bool sc1_stores, hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    static const void *const fns[2][3] = {
        {reinterpret_cast<const void *>(&kvcopy_h2d_wg_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2h_wg_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2d_wg_kernel)},
        {reinterpret_cast<const void *>(&kvcopy_h2d_wg_sc1_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2h_wg_sc1_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2d_wg_sc1_kernel)}};
    void *args[] = {(void *)&recs, (void *)&n_chunks};
    return hipExtLaunchKernel(fns[sc1_stores ? 1 : 0][dir], dim3(grid), dim3(kThreadsPerWG), args,
                              0, stream, start, stop, 0);
}

hipError_t launch_copy_pair(const ChunkRec *ra, uint32_t ca, const ChunkRec *rb, uint32_t cb,
                            uint32_t grid, bool sc1_stores, hipStream_t stream, hipEvent_t start,
                            hipEvent_t stop)
{
    uint32_t wa = pair_split(ca, cb, grid * kWavesPerWG);
    void *args[] = {(void *)&ra, (void *)&ca, (void *)&rb, (void *)&cb, (void *)&wa};
    const void *fn = sc1_stores ? reinterpret_cast<const void *>(&kvcopy_pair_kernel)
                                : reinterpret_cast<const void *>(&kvcopy_pair_nt_kernel);
    return hipExtLaunchKernel(fn, dim3(grid), dim3(kThreadsPerWG), args, 0, stream, start, stop, 0);
}

hipError_t launch_copy_inline(const InlineWork &w, uint32_t grid, int dir, bool sc1_stores,
                              hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    static const void *const fns[2][3] = {
        {reinterpret_cast<const void *>(&kvcopy_h2d_inline_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2h_inline_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2d_inline_kernel)},
        {reinterpret_cast<const void *>(&kvcopy_h2d_inline_sc1_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2h_inline_sc1_kernel),
         reinterpret_cast<const void *>(&kvcopy_d2d_inline_sc1_kernel)}};
    void *args[] = {(void *)&w};
    return hipExtLaunchKernel(fns[sc1_stores ? 1 : 0][dir], dim3(grid), dim3(kThreadsPerWG), args,
                              0, stream, start, stop, 0);
}

hipError_t launch_copy_dynamic(const ChunkRec *recs, uint32_t n_chunks, uint32_t grid, int dir,
                               uint32_t *claim, uint32_t grain, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop)
{
    static const void *const fns[3] = {reinterpret_cast<const void *>(&kvcopy_h2d_dyn_kernel),
                                       reinterpret_cast<const void *>(&kvcopy_d2h_dyn_kernel),
                                       reinterpret_cast<const void *>(&kvcopy_d2d_dyn_kernel)};
    void *args[] = {(void *)&recs, (void *)&n_chunks, (void *)&claim, (void *)&grain};
    return hipExtLaunchKernel(fns[dir], dim3(grid), dim3(kThreadsPerWG), args, 0, stream, start,
                              stop, 0);
}

}  // namespace kvc
