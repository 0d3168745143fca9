// plan.cpp -- host-side planning of a batch: validate, coalesce, chunk.
//
// Coalescing: PegaFlow issue #408 ("Kernel transfer backend causes decode
// TPOT tail spikes under concurrent KV transfers"), section "Relevant
// implementation" -- adjacent ranges are merged before submission.  The rule
// used: one pass in list order; zero sizes dropped; a range joins the one
// built so far when it continues it in both source and destination.
//
// Chunking: FreeToken issue #751 ("gather missed experts with a few TMA
// bulk-copy CTAs"), section "What we changed" -- the call's bytes are cut
// into chunks of at most 16 KiB, each inside one row, and spread over a few
// workers so that one 1 MiB row does not leave the workers of small rows idle.
// Here the chunk numbers of range i start at the exclusive prefix sum of the
// per-range chunk counts, so every range's worklist entries can be written
// independently.
#include <stdlib.h>
#include <string.h>

#include <immintrin.h>

#include <algorithm>
#include <vector>

#include "kvcopy.h"
#include "kvcopy_internal.h"

namespace kvc {

int merge_ranges(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
                 bool merge, uint64_t *osrc, uint64_t *odst, uint64_t *osize, uint64_t *m_out,
                 uint64_t *total_out)
{
    uint64_t bits = 0, total = 0, m = 0;
    bool wrap = false;
    // Current open range (not yet written) so that in-place use is safe.
    uint64_t cs = 0, cd = 0, cn = 0;
    for (uint64_t i = 0; i < n; ++i) {
        const uint64_t s = src[i], d = dst[i], z = size[i];
        bits |= s | d | z;
        if (z == 0)
            continue;
        wrap |= (s + z < s) | (d + z < d);
        total += z;
        if (cn != 0 && merge && cs + cn == s && cd + cn == d) {
            cn += z;
            continue;
        }
        if (cn != 0) {
            osrc[m] = cs;
            odst[m] = cd;
            osize[m] = cn;
            ++m;
        }
        cs = s;
        cd = d;
        cn = z;
    }
    if (cn != 0) {
        osrc[m] = cs;
        odst[m] = cd;
        osize[m] = cn;
        ++m;
    }
    *m_out = m;
    *total_out = total;
    if (bits & 7u)
        return KVCOPY_EALIGN;
    if (wrap)
        return KVCOPY_EINVAL;
    return KVCOPY_OK;
}

int check_overlap(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t m)
{
    std::vector<std::pair<uint64_t, uint64_t>> d;
    d.reserve(m);
    for (uint64_t i = 0; i < m; ++i)
        if (size[i])
            d.push_back({dst[i], dst[i] + size[i]});
    std::sort(d.begin(), d.end());
    for (size_t i = 1; i < d.size(); ++i)
        if (d[i].first < d[i - 1].second)
            return KVCOPY_EOVERLAP;
    // Destinations are now disjoint and sorted: a source overlaps one iff the
    // last destination starting before the source's end reaches past its start.
    for (uint64_t i = 0; i < m; ++i) {
        if (size[i] == 0)
            continue;
        const uint64_t lo = src[i], hi = src[i] + size[i];
        auto it = std::lower_bound(d.begin(), d.end(), std::make_pair(hi, (uint64_t)0));
        if (it != d.begin() && std::prev(it)->second > lo)
            return KVCOPY_EOVERLAP;
    }
    return KVCOPY_OK;
}

int prescan(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
            uint32_t chunk, Prescan *out)
{
    uint64_t bits = 0, total = 0, nnz = 0, bad = 0;
    for (uint64_t i = 0; i < n; ++i) {
        const uint64_t s = src[i], d = dst[i], z = size[i];
        const uint64_t t = total + z;
        bits |= s | d | z;
        bad |= (uint64_t)(s + z < s) | (uint64_t)(d + z < d) | (uint64_t)(t < total);
        total = t;
        nnz += z != 0;
    }
    if (bits & 7u)
        return KVCOPY_EALIGN;
    if (bad)
        return KVCOPY_EINVAL;
    out->nnz = nnz;
    out->total = total;
    out->bound = nnz + total / chunk;
    return KVCOPY_OK;
}

namespace {

// One record, written either through the cache or with non-temporal 8-byte
// stores (three per record).  Records bound for the pinned staging ring are
// streamed: the GPU reads them over the host link and the CPU never reads
// them back, so taking each ring line into the cache first (the
// read-for-ownership of a plain store) only costs memory traffic.  Planning
// 65,536 descriptors took 91 -> 85 us per call on an MI355X server's host
// (and 250 -> 125 us on a smaller EPYC host).  The caller orders the
// streamed stores before the launch (finish_records).
template <bool Stream>
inline void put_rec(ChunkRec *r, uint64_t s, uint64_t d, uint32_t bytes)
{
    if (Stream) {
        long long *p = reinterpret_cast<long long *>(r);
        _mm_stream_si64(p, (long long)s);
        _mm_stream_si64(p + 1, (long long)d);
        _mm_stream_si64(p + 2, (long long)bytes);   // bytes, then reserved = 0
    } else {
        *r = ChunkRec{s, d, bytes, 0};
    }
}

// The planning pass's state: validity accumulators, records written, and
// the open range (the last range, not yet written, which the next
// descriptor may still extend).
struct PassState {
    uint64_t bits = 0, bad = 0, total = 0, w = 0;
    uint64_t cs = 0, cd = 0, cn = 0;
};

// Fast path of the planning pass for the common case: a run of descriptors
// each of size 1..chunk, none continuing the one before it, none wrapping.
// Four descriptors at a time, entered with no open range: AVX2 compares
// check the sizes, the wrap and the merge rule for all four (and that the
// descriptor after them is non-empty and does not continue the fourth, so
// the fourth's range is closed too); the four records are transposed in
// registers (two unpacks, a blend and three lane permutes) and written as
// three 32-byte stores, where the scalar path makes twelve 8-byte ones.
// Returns the index of the first descriptor it did not consume; the scalar
// pass takes over from there with no open range.
template <bool Stream>
__attribute__((target("avx2"))) uint64_t fast_groups_avx2(const uint64_t *src, const uint64_t *dst,
                                                          const uint64_t *size, uint64_t i,
                                                          uint64_t n, bool merge, uint32_t chunk,
                                                          ChunkRec *out, uint64_t cap, PassState &st)
{
    const __m256i flip = _mm256_set1_epi64x((long long)0x8000000000000000ull);
    const __m256i lim = _mm256_xor_si256(_mm256_set1_epi64x((long long)chunk), flip);
    const __m256i one = _mm256_set1_epi64x(1);
    const __m256i zero = _mm256_setzero_si256();
    __m256i vbits = zero, vtotal = zero;
    // total + 4 * chunk per group must not overflow (else the scalar pass flags it)
    const uint64_t total_max = ~0ull - 4ull * chunk * (n / 4 + 1);
    uint64_t w = st.w;
    if (st.total > total_max)
        return i;
    while (i + 5 <= n && w + 4 <= cap) {
        const __m256i S = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(src + i));
        const __m256i D = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(dst + i));
        const __m256i Z = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(size + i));
        // every size in [1, chunk]: z - 1 < chunk, unsigned
        const __m256i zok = _mm256_cmpgt_epi64(lim, _mm256_xor_si256(_mm256_sub_epi64(Z, one), flip));
        const __m256i SE = _mm256_add_epi64(S, Z), DE = _mm256_add_epi64(D, Z);
        // no wrap: s + z >= s and d + z >= d, unsigned
        __m256i bad =
            _mm256_or_si256(_mm256_cmpgt_epi64(_mm256_xor_si256(S, flip), _mm256_xor_si256(SE, flip)),
                            _mm256_cmpgt_epi64(_mm256_xor_si256(D, flip), _mm256_xor_si256(DE, flip)));
        // the descriptor after each of the four: non-empty (the fourth's
        // successor; a zero size would hide which one follows) and, with
        // merging, not continuing it in both arenas
        const __m256i Zn = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(size + i + 1));
        bad = _mm256_or_si256(bad, _mm256_cmpeq_epi64(Zn, zero));
        if (merge) {
            const __m256i Sn = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(src + i + 1));
            const __m256i Dn = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(dst + i + 1));
            bad = _mm256_or_si256(bad, _mm256_and_si256(_mm256_cmpeq_epi64(SE, Sn),
                                                        _mm256_cmpeq_epi64(DE, Dn)));
        }
        if (_mm256_movemask_epi8(zok) != -1 || !_mm256_testz_si256(bad, bad))
            break;
        vbits = _mm256_or_si256(vbits, _mm256_or_si256(_mm256_or_si256(S, D), Z));
        vtotal = _mm256_add_epi64(vtotal, Z);
        // records [s0 d0 z0] [s1 d1 z1] [s2 d2 z2] [s3 d3 z3] as 16-byte
        // pairs [s0 d0][z0 s1][d1 z1] [s2 d2][z2 s3][d3 z3]
        const __m256i y0 = _mm256_unpacklo_epi64(S, D);        // [s0 d0 | s2 d2]
        const __m256i y1 = _mm256_blend_epi32(Z, S, 0xCC);     // [z0 s1 | z2 s3]
        const __m256i y2 = _mm256_unpackhi_epi64(D, Z);        // [d1 z1 | d3 z3]
        const __m256i r0 = _mm256_permute2x128_si256(y0, y1, 0x20);
        const __m256i r1 = _mm256_permute2x128_si256(y2, y0, 0x30);
        const __m256i r2 = _mm256_permute2x128_si256(y1, y2, 0x31);
        __m256i *o = reinterpret_cast<__m256i *>(out + w);
        if (Stream && (reinterpret_cast<uintptr_t>(o) & 31u) == 0) {
            _mm256_stream_si256(o, r0);
            _mm256_stream_si256(o + 1, r1);
            _mm256_stream_si256(o + 2, r2);
        } else if (Stream) {
            // not 32-byte aligned (w not a multiple of 4 on a 32-byte aligned
            // ring): still only non-temporal stores, 8 bytes at a time.  A
            // cached store into lines that non-temporal stores are filling
            // flushes their write-combining buffers: measured on a 2.7 GHz
            // Xeon, 65,536 mixed-size descriptors planned in 1.1 ms with
            // cached stores here against 0.6 ms without.
            alignas(32) long long q[12];
            _mm256_store_si256(reinterpret_cast<__m256i *>(q), r0);
            _mm256_store_si256(reinterpret_cast<__m256i *>(q + 4), r1);
            _mm256_store_si256(reinterpret_cast<__m256i *>(q + 8), r2);
            long long *o8 = reinterpret_cast<long long *>(o);
            for (int k = 0; k < 12; ++k)
                _mm_stream_si64(o8 + k, q[k]);
        } else {
            _mm256_storeu_si256(o, r0);
            _mm256_storeu_si256(o + 1, r1);
            _mm256_storeu_si256(o + 2, r2);
        }
        w += 4;
        i += 4;
    }
    alignas(32) uint64_t b[4], t[4];
    _mm256_store_si256(reinterpret_cast<__m256i *>(b), vbits);
    _mm256_store_si256(reinterpret_cast<__m256i *>(t), vtotal);
    st.bits |= b[0] | b[1] | b[2] | b[3];
    st.total += t[0] + t[1] + t[2] + t[3];
    st.w = w;
    return i;
}

bool have_avx2()
{
    static const bool yes = __builtin_cpu_supports("avx2");
    return yes;
}

template <bool Stream, bool Fast>
int build_checked_impl(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
                       bool merge, uint32_t chunk, ChunkRec *out, uint64_t cap, uint64_t *n_chunks)
{
    PassState st;
    auto close = [&]() {
        if (st.cn <= chunk) {   // the common case: one chunk per range
            if (st.w < cap)
                put_rec<Stream>(out + st.w, st.cs, st.cd, (uint32_t)st.cn);
            ++st.w;
            return;
        }
        // Count arithmetically and write only what fits: an invalid list (a
        // size that wraps, say) is rejected after the pass, and must not cost
        // a loop over its chunks first.
        const uint64_t k = st.cn / chunk + (st.cn % chunk != 0);
        const uint64_t room = st.w < cap ? cap - st.w : 0;
        const uint64_t put = k < room ? k : room;
        for (uint64_t j = 0; j < put; ++j) {
            const uint64_t off = j * chunk, left = st.cn - off;
            put_rec<Stream>(out + st.w + j, st.cs + off, st.cd + off,
                            (uint32_t)(left < chunk ? left : chunk));
        }
        st.w += k;
    };
    // After a group the fast path declined, go on scalar for a while, for
    // twice as long after each further decline in a row (up to 1,024
    // descriptors), so that stretches where it does not apply cost little.
    uint64_t retry = 0;
    unsigned declined = 0;
    for (uint64_t i = 0; i < n;) {
        if (Fast && i >= retry) {
            // Close the open range early when descriptor i (non-empty) does
            // not continue it, so the fast path starts with no open range.
            const uint64_t zi = size[i];
            if (st.cn != 0 && zi != 0 &&
                !(merge && st.cs + st.cn == src[i] && st.cd + st.cn == dst[i])) {
                close();
                st.cn = 0;
            }
            if (st.cn == 0) {
                const uint64_t j = fast_groups_avx2<Stream>(src, dst, size, i, n, merge, chunk, out,
                                                            cap, st);
                if (j == i) {
                    retry = i + (4ull << declined);
                    declined += declined < 8;
                } else {
                    declined = 0;
                }
                i = j;
                if (i >= n)
                    break;
            }
        }
        const uint64_t s = src[i], d = dst[i], z = size[i];
        ++i;
        const uint64_t t = st.total + z;
        st.bits |= s | d | z;
        st.bad |= (uint64_t)(s + z < s) | (uint64_t)(d + z < d) | (uint64_t)(t < st.total);
        st.total = t;
        if (z == 0)
            continue;
        if (merge && st.cn != 0 && st.cs + st.cn == s && st.cd + st.cn == d) {
            st.cn += z;
            continue;
        }
        if (st.cn != 0)
            close();
        st.cs = s;
        st.cd = d;
        st.cn = z;
    }
    if (st.cn != 0)
        close();
    if (st.bits & 7u)
        return KVCOPY_EALIGN;
    if (st.bad)
        return KVCOPY_EINVAL;
    *n_chunks = st.w;
    return KVCOPY_OK;
}

}  // namespace

// Whether build_checked takes the vector path for this list: the host has
// AVX2 and, of the list's first 64 descriptors, at least 7 in 8 are
// single-chunk (size in [1, chunk]) and do not continue their predecessor.
// Lists of one block size (KV pages, say) pass; mixed sizes with merges do
// not, and for them the scalar pass alone is faster: measured on a 2.7 GHz
// Xeon, 65,536 mixed 4-28 KiB descriptors with 25% merges planned in
// 0.52 ms by the scalar pass against 0.59 ms with the vector path compiled
// in and rarely taken.
bool planner_vector_path(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
                         bool merge, uint32_t chunk)
{
    if (!have_avx2())
        return false;
    const uint64_t m = n < 64 ? n : 64;
    uint64_t good = 0;
    for (uint64_t i = 0; i < m; ++i) {
        const bool single = size[i] - 1 < chunk;   // unsigned: size in [1, chunk]
        const bool cont = merge && i > 0 && src[i - 1] + size[i - 1] == src[i] &&
                          dst[i - 1] + size[i - 1] == dst[i];
        good += single && !cont;
    }
    return m >= 16 && good * 8 >= m * 7;
}

int build_checked(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
                  bool merge, uint32_t chunk, ChunkRec *out, uint64_t cap, uint64_t *n_chunks,
                  bool stream)
{
    if (planner_vector_path(src, dst, size, n, merge, chunk))
        return stream ? build_checked_impl<true, true>(src, dst, size, n, merge, chunk, out, cap, n_chunks)
                      : build_checked_impl<false, true>(src, dst, size, n, merge, chunk, out, cap, n_chunks);
    return stream ? build_checked_impl<true, false>(src, dst, size, n, merge, chunk, out, cap, n_chunks)
                  : build_checked_impl<false, false>(src, dst, size, n, merge, chunk, out, cap, n_chunks);
}

void finish_records()
{
    _mm_sfence();
}

uint64_t build_worklist(const uint64_t *src, const uint64_t *dst, const uint64_t *size, uint64_t n,
                        bool merge, uint32_t chunk, ChunkRec *out)
{
    uint64_t w = 0;
    (void)build_checked(src, dst, size, n, merge, chunk, out, ~0ull, &w);
    return w;
}

// Destination order for D2D gathers of random blocks, made on the host
// when the worklist is read in place from the ring (with an upload the GPU
// groups it, order_kernel.hip): with the worklist in list order, the
// chunks that the GPU has in flight at any moment write all over HBM;
// grouped by destination region, the wavefronts that the dispatcher starts
// together write into a narrow band of rows.  Measured on MI355X with one
// wavefront per chunk (65,536 random 4 KiB blocks between two 1 GiB pools,
// calls over 8 distinct batches): regions of 1, 4, 16 and 64 MiB and a full
// sort by destination all gave 100.8-103 us against 107 us in list order,
// so the regions are 64 MiB, 16 of them: a stable counting sort with 16
// output streams, which the host's prefetchers follow (a 4 MiB grouping,
// 256 streams, cost 20 us more per 65,536 records on the MI355X host for no
// gain with this loop).  The records are written with ordinary (cached)
// stores: non-temporal stores scattered over the streams each flush a partly
// filled write-combining buffer, which measured 20 times slower.
void order_by_dst(const ChunkRec *in, uint64_t n, ChunkRec *out)
{
    uint64_t at[kDstBuckets] = {};
    for (uint64_t i = 0; i < n; ++i)
        ++at[(in[i].dst >> kDstRegionShift) & (kDstBuckets - 1)];
    uint64_t acc = 0;
    for (uint32_t b = 0; b < kDstBuckets; ++b) {
        const uint64_t c = at[b];
        at[b] = acc;
        acc += c;
    }
    for (uint64_t i = 0; i < n; ++i) {
        const ChunkRec &r = in[i];
        out[at[(r.dst >> kDstRegionShift) & (kDstBuckets - 1)]++] = r;
    }
}

uint64_t chunk_prefix(const uint64_t *size, uint64_t m, uint32_t chunk, uint64_t *begin)
{
    uint64_t acc = 0;
    for (uint64_t i = 0; i < m; ++i) {
        begin[i] = acc;
        acc += size[i] / chunk + (size[i] % chunk != 0);
    }
    begin[m] = acc;
    return acc;
}

void emit_chunks(const uint64_t *src, const uint64_t *dst, const uint64_t *size,
                 const uint64_t *begin, uint64_t m, uint32_t chunk, ChunkRec *out)
{
    for (uint64_t i = 0; i < m; ++i) {
        ChunkRec *r = out + begin[i];
        const uint64_t s = src[i], d = dst[i], z = size[i];
        if (z <= chunk) {   // the common case: one chunk per range
            r->src = s;
            r->dst = d;
            r->bytes = (uint32_t)z;
            r->reserved = 0;
            continue;
        }
        for (uint64_t off = 0; off < z; off += chunk, ++r) {
            const uint64_t left = z - off;
            r->src = s + off;
            r->dst = d + off;
            r->bytes = (uint32_t)(left < chunk ? left : chunk);
            r->reserved = 0;
        }
    }
}

bool env_validate(bool *bad)
{
    const char *v = getenv("KVCOPY_VALIDATE");
    *bad = false;
    if (v == nullptr || strcmp(v, "0") == 0)
        return false;
    if (strcmp(v, "1") == 0)
        return true;
    *bad = true;
    return false;
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvcopy_coalesce(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes,
                               uint64_t n, uint64_t *out_src, uint64_t *out_dst,
                               uint64_t *out_sizes, uint64_t *out_n)
{
    if (out_n == nullptr)
        return KVCOPY_EINVAL;
    if (n == 0) {
        *out_n = 0;
        return KVCOPY_OK;
    }
    if (!src || !dst || !sizes || !out_src || !out_dst || !out_sizes)
        return KVCOPY_EINVAL;
    // Same pass as the batch planner; alignment is not this call's concern.
    uint64_t m = 0, total = 0;
    (void)merge_ranges(src, dst, sizes, n, true, out_src, out_dst, out_sizes, &m, &total);
    *out_n = m;
    return KVCOPY_OK;
}

extern "C" int kvcopy_plan(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes,
                           uint64_t n, uint32_t chunk_bytes, kvcopy_plan_t *out)
{
    if (out == nullptr)
        return KVCOPY_EINVAL;
    memset(out, 0, sizeof(*out));
    if (chunk_bytes == 0)
        chunk_bytes = KVCOPY_CHUNK_DEFAULT;
    if ((chunk_bytes & 15u) || chunk_bytes > KVCOPY_CHUNK_MAX)
        return KVCOPY_EINVAL;
    if (n > KVCOPY_MAX_DESCS || (n > 0 && (!src || !dst || !sizes)))
        return KVCOPY_EINVAL;
    bool bad_env = false;
    const bool validate = env_validate(&bad_env);
    if (bad_env)
        return KVCOPY_EINVAL;

    // One allocation holds src, dst, size (n each) and chunk_begin (n + 1).
    uint64_t *buf = (uint64_t *)malloc(sizeof(uint64_t) * (4 * n + 1));
    if (buf == nullptr)
        return KVCOPY_ENOMEM;
    uint64_t *ms = buf, *md = buf + n, *mz = buf + 2 * n, *mb = buf + 3 * n;
    uint64_t m = 0, total = 0;
    int rc = merge_ranges(src, dst, sizes, n, true, ms, md, mz, &m, &total);
    if (rc == KVCOPY_OK && validate)
        rc = check_overlap(ms, md, mz, m);
    if (rc != KVCOPY_OK) {
        free(buf);
        return rc;
    }
    const uint64_t chunks = chunk_prefix(mz, m, chunk_bytes, mb);
    if (chunks > KVCOPY_MAX_CHUNKS) {
        free(buf);
        return KVCOPY_EINVAL;
    }
    out->n_in = n;
    out->n_merged = m;
    out->n_chunks = chunks;
    out->total_bytes = total;
    out->chunk_bytes = chunk_bytes;
    out->src = ms;
    out->dst = md;
    out->size = mz;
    out->chunk_begin = mb;
    return KVCOPY_OK;
}

extern "C" void kvcopy_plan_free(kvcopy_plan_t *plan)
{
    if (plan == nullptr)
        return;
    free((void *)plan->src);   // the arrays share one allocation starting at src
    memset(plan, 0, sizeof(*plan));
}
