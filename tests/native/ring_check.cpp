// The staging ring never hands out bytes that a still-running kernel may read.
//
// Simulated events: each committed region gets a completion time on a
// virtual clock; kernels on different streams complete out of order.  poll()
// reports completion against the clock, wait() advances the clock to the
// event's completion.  After every reserve() the new region must lie inside
// the ring and overlap no region whose event has not completed yet.
#include <cstdio>
#include <random>
#include <vector>

#include "staging_ring.h"

struct Sim {
    std::vector<double> done_at;   // event id -> completion time
    double now = 0;
    int waits = 0;
};

struct FakeOps {
    Sim *sim;
    int poll(int ev) { return sim->done_at[ev] <= sim->now ? 1 : 0; }
    int wait(int ev)
    {
        if (sim->done_at[ev] > sim->now)
            sim->now = sim->done_at[ev];
        ++sim->waits;
        return 0;
    }
    void recycle(int) {}
};

int main()
{
    std::mt19937_64 rng(7);
    long checks = 0;
    for (int trial = 0; trial < 200; ++trial) {
        Sim sim;
        kvc::StagingRing<int, FakeOps> ring(FakeOps{&sim});
        const uint64_t cap = 256 * (64 + rng() % 4096);
        ring.reset(cap);
        struct Live { uint64_t b, e; int ev; };
        std::vector<Live> live;
        double stream_end[3] = {0, 0, 0};
        for (int call = 0; call < 3000; ++call) {
            const uint64_t need = 256 * (1 + rng() % (cap / 256 / 4));
            uint64_t off = ~0ull;
            if (ring.reserve(need, &off) != 0) {
                printf("reserve failed\n");
                return 1;
            }
            if (off + need > cap || off % 256) {
                printf("trial %d call %d: region [%lu, %lu) outside ring of %lu\n", trial, call,
                       (unsigned long)off, (unsigned long)(off + need), (unsigned long)cap);
                return 1;
            }
            for (const Live &l : live) {
                if (sim.done_at[l.ev] > sim.now && off < l.e && l.b < off + need) {
                    printf("trial %d call %d: [%lu, %lu) overlaps running [%lu, %lu)\n", trial, call,
                           (unsigned long)off, (unsigned long)(off + need), (unsigned long)l.b,
                           (unsigned long)l.e);
                    return 1;
                }
                ++checks;
            }
            const uint64_t used = 256 * (1 + rng() % (need / 256));
            const int s = (int)(rng() % 3);                      // the caller's stream
            const double start = stream_end[s] > sim.now ? stream_end[s] : sim.now;
            stream_end[s] = start + 1 + (double)(rng() % 50);   // kernels on one stream run in order
            const int ev = (int)sim.done_at.size();
            sim.done_at.push_back(stream_end[s]);
            ring.commit(off, used, ev);
            live.push_back({off, off + used, ev});
            sim.now += (double)(rng() % 8);                     // host time between calls
            if (live.size() > 64)
                live.erase(live.begin(), live.begin() + 32);    // old entries: completed long ago
        }
    }
    printf("ok %ld overlap checks\n", checks);
    return 0;
}
