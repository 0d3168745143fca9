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
    printf("ok %d cases\n", cases);
    return 0;
}
