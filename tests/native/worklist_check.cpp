// The batch path's fused planner (build_worklist) must write exactly the
// records that the step-by-step planner (merge_ranges -> chunk_prefix ->
// emit_chunks) gives, for random descriptor lists with zero sizes, chains of
// adjacent ranges, and ranges longer than a chunk; prescan's bound must hold.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "kvcopy.h"
#include "kvcopy_internal.h"

using namespace kvc;

int main(int argc, char **argv)
{
    const int trials = argc > 1 ? atoi(argv[1]) : 1500;   // fewer under the sanitizers
    std::mt19937_64 rng(12345);
    const uint32_t chunks[] = {16, 64, 4096, 16384, 65536};
    int cases = 0;
    for (int trial = 0; trial < trials; ++trial) {
        const uint64_t n = rng() % 300;
        const uint32_t chunk = chunks[rng() % 5];
        std::vector<uint64_t> s(n), d(n), z(n);
        uint64_t cs = 1ull << 32, cd = 1ull << 40;
        for (uint64_t i = 0; i < n; ++i) {
            const int kind = (int)(rng() % 4);
            z[i] = (rng() % 5 == 0) ? 0 : 8 * (1 + rng() % (kind == 0 ? 40000 : 3000));
            if (kind == 1 && i > 0) {          // continue the previous descriptor in both arenas
                s[i] = s[i - 1] + z[i - 1];
                d[i] = d[i - 1] + z[i - 1];
            } else {
                cs += 8 * (1 + rng() % 1000) + z[i];
                cd += 8 * (1 + rng() % 1000) + z[i];
                s[i] = cs;
                d[i] = cd;
            }
        }
        for (int merge = 0; merge < 2; ++merge) {
            Prescan pre;
            if (prescan(s.data(), d.data(), z.data(), n, chunk, &pre) != KVCOPY_OK) {
                printf("prescan rejected a valid list\n");
                return 1;
            }
            std::vector<uint64_t> ms(n + 1), md(n + 1), mz(n + 1), mb(n + 2);
            uint64_t m = 0, total = 0;
            merge_ranges(s.data(), d.data(), z.data(), n, merge, ms.data(), md.data(), mz.data(), &m,
                         &total);
            const uint64_t c = chunk_prefix(mz.data(), m, chunk, mb.data());
            std::vector<ChunkRec> ref(c + 1), got(pre.bound + 1);
            emit_chunks(ms.data(), md.data(), mz.data(), mb.data(), m, chunk, ref.data());
            const uint64_t c2 = build_worklist(s.data(), d.data(), z.data(), n, merge, chunk, got.data());
            if (c2 != c || c > pre.bound || total != pre.total ||
                (c && memcmp(ref.data(), got.data(), c * sizeof(ChunkRec)) != 0)) {
                printf("mismatch: trial %d merge %d n %lu chunk %u: %lu vs %lu records (bound %lu)\n",
                       trial, merge, (unsigned long)n, chunk, (unsigned long)c, (unsigned long)c2,
                       (unsigned long)pre.bound);
                return 1;
            }
            // The checked pass with a short room: same count, same prefix,
            // with plain and with streamed stores.
            for (uint64_t cap : {(uint64_t)0, c / 2, c, c + 3})
            for (bool streamed : {false, true}) {
                std::vector<ChunkRec> part(cap + 1);
                memset(part.data(), 0xA5, part.size() * sizeof(ChunkRec));
                uint64_t need = ~0ull;
                const int rc = build_checked(s.data(), d.data(), z.data(), n, merge, chunk,
                                             part.data(), cap, &need, streamed);
                finish_records();
                const uint64_t wrote = cap < c ? cap : c;
                if (rc != KVCOPY_OK || need != c ||
                    (wrote && memcmp(ref.data(), part.data(), wrote * sizeof(ChunkRec)) != 0)) {
                    printf("build_checked: trial %d cap %lu streamed %d: rc %d need %lu want %lu\n",
                           trial, (unsigned long)cap, (int)streamed, rc, (unsigned long)need,
                           (unsigned long)c);
                    return 1;
                }
                // nothing written past the room
                const unsigned char *tail = reinterpret_cast<const unsigned char *>(part.data() + wrote);
                for (size_t b = 0; b < (part.size() - wrote) * sizeof(ChunkRec); ++b)
                    if (tail[b] != 0xA5) {
                        printf("build_checked: trial %d cap %lu streamed %d wrote past its room\n",
                               trial, (unsigned long)cap, (int)streamed);
                        return 1;
                    }
            }
            ++cases;
        }
        // Broken copies of the list: build_checked rejects them as prescan does.
        if (n > 0) {
            const uint64_t i = rng() % n;
            for (int k = 0; k < 4; ++k) {
                std::vector<uint64_t> s2 = s, d2 = d, z2 = z;
                if (k == 0) s2[i] += 4;                       // misaligned source
                if (k == 1) z2[i] = 12;                       // size not a multiple of 8
                if (k == 2) d2[i] = ~0ull - 7, z2[i] = 64;    // destination range wraps
                if (k == 3) z2[i] = ~0ull - 7;                // size wraps the source range
                Prescan p2;
                const int want = prescan(s2.data(), d2.data(), z2.data(), n, chunk, &p2);
                std::vector<ChunkRec> tmp(8);
                uint64_t need = 0;
                const int got = build_checked(s2.data(), d2.data(), z2.data(), n, true, chunk,
                                              tmp.data(), 8, &need);
                if (want == KVCOPY_OK || got != want) {
                    printf("build_checked error: trial %d kind %d: %d vs prescan %d\n", trial, k,
                           got, want);
                    return 1;
                }
            }
        }
    }
    // Runs of block descriptors (the planner's vector fast path): mostly
    // non-adjacent 4 KiB blocks, with rare zero sizes, chains of adjacent
    // blocks, ranges longer than a chunk and misaligned entries, planned
    // into outputs at every 8-byte offset within 32 bytes and with rooms
    // that end mid-list, plain and streamed; the records must equal the
    // step-by-step planner's.
    int vector_lists = 0, block_lists = 0;
    for (int trial = 0; trial < trials; ++trial) {
        const uint64_t n = 5 + rng() % 2000;
        const uint32_t chunk = (rng() % 3 == 0) ? 4096 : 16384;
        std::vector<uint64_t> s(n), d(n), z(n);
        const int rare = 1 + (int)(rng() % 200);
        for (uint64_t i = 0; i < n; ++i) {
            z[i] = 4096;
            const int r = (int)(rng() % 1000);
            if (r < rare / 4)
                z[i] = 0;
            else if (r < rare / 2)
                z[i] = 8 * (1 + rng() % 8000);
            if (i > 0 && r >= rare / 2 && r < rare) {
                s[i] = s[i - 1] + z[i - 1];
                d[i] = d[i - 1] + z[i - 1];
            } else {
                s[i] = (1ull << 36) + (rng() % (1u << 20)) * 4096 + (r == 999 ? 12 : 0);
                d[i] = (1ull << 40) + (rng() % (1u << 20)) * 4096;
            }
        }
        for (int merge = 0; merge < 2; ++merge) {
            ++block_lists;
            vector_lists += planner_vector_path(s.data(), d.data(), z.data(), n, merge, chunk);
            std::vector<uint64_t> ms(n + 1), md(n + 1), mz(n + 1), mb(n + 2);
            uint64_t m = 0, total = 0;
            const int mrc = merge_ranges(s.data(), d.data(), z.data(), n, merge, ms.data(), md.data(),
                                         mz.data(), &m, &total);
            const uint64_t c = chunk_prefix(mz.data(), m, chunk, mb.data());
            std::vector<ChunkRec> ref(c + 1);
            emit_chunks(ms.data(), md.data(), mz.data(), mb.data(), m, chunk, ref.data());
            for (int shift = 0; shift < 4; ++shift)
            for (uint64_t cap : {c, c / 3, c + 5})
            for (bool streamed : {false, true}) {
                std::vector<unsigned char> raw((cap + 8) * sizeof(ChunkRec) + 64, 0xA5);
                uintptr_t base = (reinterpret_cast<uintptr_t>(raw.data()) + 31) & ~(uintptr_t)31;
                ChunkRec *part = reinterpret_cast<ChunkRec *>(base + 8 * shift);
                uint64_t need = ~0ull;
                const int rc = build_checked(s.data(), d.data(), z.data(), n, merge, chunk, part, cap,
                                             &need, streamed);
                finish_records();
                if (rc != mrc) {
                    printf("fast path: trial %d: rc %d, merge_ranges %d\n", trial, rc, mrc);
                    return 1;
                }
                if (rc != KVCOPY_OK)
                    continue;
                const uint64_t wrote = cap < c ? cap : c;
                if (need != c || (wrote && memcmp(ref.data(), part, wrote * sizeof(ChunkRec)) != 0)) {
                    printf("fast path: trial %d merge %d shift %d cap %llu streamed %d: %llu records,"
                           " want %llu\n", trial, merge, shift, (unsigned long long)cap, (int)streamed,
                           (unsigned long long)need, (unsigned long long)c);
                    return 1;
                }
                const unsigned char *tail = reinterpret_cast<const unsigned char *>(part + wrote);
                for (size_t b = 0; b < 8 * sizeof(ChunkRec); ++b)
                    if (tail[b] != 0xA5) {
                        printf("fast path: trial %d wrote past its room\n", trial);
                        return 1;
                    }
            }
            ++cases;
        }
    }
    // On an AVX2 host most of these lists must take the vector path, or the
    // block above would not test it.
    if (__builtin_cpu_supports("avx2") && vector_lists * 2 < block_lists) {
        printf("fast path: only %d of %d block lists took the vector path\n", vector_lists,
               block_lists);
        return 1;
    }
    // Mixed sizes with merges (the H2D mixed-size workload's shape) take the
    // scalar pass.
    {
        std::vector<uint64_t> s(4096), d(4096), z(4096);
        for (uint64_t i = 0; i < 4096; ++i) {
            z[i] = 8 * (512 + rng() % 3072);                  // 4-28 KiB
            const bool cont = i > 0 && rng() % 4 == 0;
            s[i] = cont ? s[i - 1] + z[i - 1] : (1ull << 36) + (rng() % (1u << 20)) * 32768;
            d[i] = cont ? d[i - 1] + z[i - 1] : (1ull << 40) + (rng() % (1u << 20)) * 32768;
        }
        if (planner_vector_path(s.data(), d.data(), z.data(), 4096, true, 16384)) {
            printf("fast path: a mixed-size list with merges took the vector path\n");
            return 1;
        }
    }
    // The default copy-loop choice: pipelined only for D2D grids of at most
    // 256 workgroups in which every wavefront has at least two chunks.
    struct { int dir; uint32_t grid; uint64_t chunks; bool want; } pol[] = {
        {KVCOPY_H2D, 1, 8, false},     {KVCOPY_H2D, 4, 32, false},     {KVCOPY_D2H, 4, 16384, false},
        {KVCOPY_D2H, 128, 16384, false}, {KVCOPY_D2D, 1, 8, true},     {KVCOPY_D2D, 1, 7, false},
        {KVCOPY_D2D, 256, 2048, true}, {KVCOPY_D2D, 256, 2047, false}, {KVCOPY_D2D, 257, 65536, false},
        {KVCOPY_D2D, 64, 65536, true},
    };
    for (const auto &c : pol) {
        if (pipeline_pays(c.dir, c.grid, c.chunks) != c.want) {
            printf("pipeline_pays(%d, %u, %llu) != %d\n", c.dir, c.grid,
                   (unsigned long long)c.chunks, (int)c.want);
            return 1;
        }
    }
    // Dynamic claims: about four claims per wavefront, between 1 and 64 chunks.
    struct { uint64_t chunks; uint32_t grid; uint32_t want; } gr[] = {
        {1024, 256, 1}, {16384, 128, 8}, {16384, 1, 64}, {65536, 16384, 1}, {3, 1, 1},
        {4096, 4, 64}, {2048, 4, 32},
    };
    for (const auto &c : gr) {
        if (claim_grain(c.chunks, c.grid) != c.want) {
            printf("claim_grain(%llu, %u) = %u, want %u\n", (unsigned long long)c.chunks, c.grid,
                   claim_grain(c.chunks, c.grid), c.want);
            return 1;
        }
    }
    // Pair launches: wavefronts for list a in proportion to the chunk counts,
    // rounded to nearest, at least one for each non-empty list.
    struct { uint64_t ca, cb; uint32_t nw, want; } sp[] = {
        {16384, 16384, 256, 128}, {0, 5, 4, 0}, {5, 0, 4, 4}, {1, 100000, 4, 1},
        {100000, 1, 4, 3}, {3, 1, 256, 192}, {1, 3, 256, 64}, {1, 1, 4, 2}, {1, 2, 4, 1},
        {2, 1, 4, 3}, {700, 37, 16, 15}, {37, 700, 16, 1}, {0xFFFFFFFFull, 0xFFFFFFFFull, 8, 4},
    };
    for (const auto &c : sp) {
        if (pair_split(c.ca, c.cb, c.nw) != c.want) {
            printf("pair_split(%llu, %llu, %u) = %u, want %u\n", (unsigned long long)c.ca,
                   (unsigned long long)c.cb, c.nw, pair_split(c.ca, c.cb, c.nw), c.want);
            return 1;
        }
    }
    for (uint32_t nw = 4; nw <= 64; nw += 4)   // every split is a valid partition
        for (uint64_t ca = 0; ca <= 40; ++ca)
            for (uint64_t cb = ca == 0 ? 1 : 0; cb <= 40; ++cb) {   // both empty: no launch
                const uint32_t wa = pair_split(ca, cb, nw);
                const bool ok = wa <= nw && (ca == 0 || wa >= 1) && (cb == 0 || wa <= nw - 1) &&
                                (ca != 0 || wa == 0) && (cb != 0 || wa == nw);
                if (!ok) {
                    printf("pair_split(%llu, %llu, %u) = %u is not a valid split\n",
                           (unsigned long long)ca, (unsigned long long)cb, nw, wa);
                    return 1;
                }
            }
    // Grid sizes at the documented limits: one wavefront per chunk, never
    // more than kMaxGrid workgroups (a launch must stay under 2^32
    // work-items), and a dynamic loop's claim counter cannot wrap: its
    // largest value is (claims below n + one overshooting claim per
    // wavefront) x grain.
    struct { uint64_t chunks; int cap; uint32_t want; } gf[] = {
        {1, 0, 1}, {4, 0, 1}, {5, 0, 2}, {1024, 0, 256}, {1024, 16, 16}, {1024, 300, 256},
        {1ull << 24, 0, 1u << 22}, {(1ull << 24) + 4, 0, 1u << 22}, {1ull << 26, 0, 1u << 22},
        {KVCOPY_MAX_CHUNKS, 0, 1u << 22}, {KVCOPY_MAX_CHUNKS, 0x7fffffff, 1u << 22},
        {KVCOPY_MAX_CHUNKS, 1000, 1000}, {KVCOPY_MAX_CHUNKS, 1, 1},
    };
    for (const auto &c : gf) {
        const uint32_t g = grid_for(c.chunks, c.cap);
        if (g != c.want) {
            printf("grid_for(%llu, %d) = %u, want %u\n", (unsigned long long)c.chunks, c.cap, g,
                   c.want);
            return 1;
        }
    }
    for (uint64_t chunks : {(uint64_t)1, (uint64_t)1000, (uint64_t)1 << 20, (uint64_t)1 << 26,
                            KVCOPY_MAX_CHUNKS})
        for (int cap : {0, 1, 7, 256, 65536, 0x7fffffff}) {
            const uint32_t g = grid_for(chunks, cap);
            const uint64_t nw = (uint64_t)g * kWavesPerWG;
            const uint64_t grain = claim_grain(chunks, g);
            const uint64_t top = ((chunks + grain - 1) / grain + nw) * grain;
            if (g == 0 || g > kMaxGrid || (uint64_t)g * kThreadsPerWG >= (1ull << 32) ||
                grain < 1 || grain > 64 || top >= (1ull << 32)) {
                printf("limits: chunks %llu cap %d: grid %u grain %llu top %llu\n",
                       (unsigned long long)chunks, cap, g, (unsigned long long)grain,
                       (unsigned long long)top);
                return 1;
            }
        }
    // Destination order (host): a permutation of the records, grouped by
    // 64 MiB destination region in key order, list order kept within a
    // region.  Each record carries its list position in `reserved` (the sort
    // moves whole records); nothing past the output is written.
    for (int trial = 0; trial < 204; ++trial) {
        const uint64_t n = trial < 200 ? rng() % 3000 : 70000 + rng() % 70000;
        std::vector<ChunkRec> in(n), out(n + 1);
        for (uint64_t i = 0; i < n; ++i)
            in[i] = ChunkRec{rng() & ~7ull, (rng() % (3ull << 30)) & ~7ull,
                             (uint32_t)(8 * (1 + rng() % 2048)), (uint32_t)i};
        memset(out.data(), 0x5A, out.size() * sizeof(ChunkRec));
        order_by_dst(in.data(), n, out.data());
        std::vector<int> seen(n, 0);
        for (uint64_t k = 0; k < n; ++k) {
            const uint64_t i = out[k].reserved;
            if (i >= n || seen[i]++ || memcmp(&out[k], &in[i], sizeof(ChunkRec)) != 0) {
                printf("order_by_dst: n %llu slot %llu is not a distinct input record\n",
                       (unsigned long long)n, (unsigned long long)k);
                return 1;
            }
            if (k > 0) {
                const uint32_t b = (uint32_t)((out[k].dst >> kDstRegionShift) & (kDstBuckets - 1));
                const uint32_t bp =
                    (uint32_t)((out[k - 1].dst >> kDstRegionShift) & (kDstBuckets - 1));
                if (bp > b || (bp == b && out[k - 1].reserved > out[k].reserved)) {
                    printf("order_by_dst: n %llu slots %llu-%llu out of order\n",
                           (unsigned long long)n, (unsigned long long)k - 1,
                           (unsigned long long)k);
                    return 1;
                }
            }
        }
        const unsigned char *tail = reinterpret_cast<const unsigned char *>(out.data() + n);
        for (size_t b = 0; b < sizeof(ChunkRec); ++b)
            if (tail[b] != 0x5A) {
                printf("order_by_dst wrote past its output (n %llu)\n", (unsigned long long)n);
                return 1;
            }
    }
    printf("ok %d cases\n", cases);
    return 0;
}
