// The batch path's fused planner (build_worklist) must write exactly the
// records that the step-by-step planner (merge_ranges -> chunk_prefix ->
// emit_chunks) gives, for random descriptor lists with zero sizes, chains of
// adjacent ranges, and ranges longer than a chunk; prescan's bound must hold.
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "kvcopy.h"
#include "kvcopy_internal.h"

using namespace kvc;

int main()
{
    std::mt19937_64 rng(12345);
    const uint32_t chunks[] = {16, 64, 4096, 16384, 65536};
    int cases = 0;
    for (int trial = 0; trial < 3000; ++trial) {
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
            ++cases;
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
    printf("ok %d cases\n", cases);
    return 0;
}
