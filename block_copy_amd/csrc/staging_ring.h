// staging_ring.h -- byte-range allocator of the worklist staging ring.
//
// Each copy call takes one contiguous region of a fixed-size ring; the
// region stays in use until the kernel that reads it has completed, which an
// event (of type Ev) reports.  Regions are handed out in ring order, so the
// in-flight list is FIFO and the oldest region is always the one in the way.
// Independent of HIP: `Ops` supplies
//   int poll(Ev)      1 = completed, 0 = still running, < 0 = error code
//   int wait(Ev)      0 = completed (after blocking),   < 0 = error code
//   void recycle(Ev)  the event may be reused
// so the allocation logic can be exercised on the CPU with simulated events.
#pragma once

#include <stdint.h>

#include <deque>

namespace kvc {

template <class Ev, class Ops>
class StagingRing {
public:
    struct Region {
        uint64_t begin, end;
        Ev ev;
    };

    explicit StagingRing(Ops ops = Ops()) : ops_(ops) {}

    uint64_t capacity() const { return cap_; }
    bool idle() const { return inflight_.empty(); }
    const std::deque<Region> &inflight() const { return inflight_; }

    // Forget every region (all must have completed: call drain() first) and
    // adopt a new capacity.
    void reset(uint64_t cap)
    {
        cap_ = cap;
        head_ = 0;
        inflight_.clear();
    }

    // Waits for and retires every in-flight region.
    int drain()
    {
        while (!inflight_.empty()) {
            const int rc = retire_front(true);
            if (rc < 0)
                return rc;
        }
        return 0;
    }

    // Finds `need` bytes (need <= capacity) at the head, or at 0 when the
    // tail end of the ring is too short, retiring completed regions on the
    // way and waiting for running ones only when they are in the way.
    int reserve(uint64_t need, uint64_t *off)
    {
        while (!inflight_.empty()) {   // retire what has finished, without waiting
            const int rc = retire_front(false);
            if (rc < 0)
                return rc;
            if (rc == 0)
                break;
        }
        for (;;) {
            if (inflight_.empty()) {
                *off = 0;
                return 0;
            }
            const uint64_t tail = inflight_.front().begin;
            if (head_ > tail) {           // used [tail, head): free [head, cap) and [0, tail)
                if (head_ + need <= cap_) {
                    *off = head_;
                    return 0;
                }
                if (need <= tail) {
                    *off = 0;
                    return 0;
                }
            } else if (head_ < tail) {    // used wraps: free [head, tail)
                if (head_ + need <= tail) {
                    *off = head_;
                    return 0;
                }
            }                             // head == tail: every byte is in use
            const int rc = retire_front(true);
            if (rc < 0)
                return rc;
        }
    }

    // Records that [off, off + used) is in use until `ev` completes.
    // `off` must come from the last reserve() and used <= the size reserved.
    void commit(uint64_t off, uint64_t used, Ev ev)
    {
        inflight_.push_back(Region{off, off + used, ev});
        head_ = off + used;
    }

private:
    int retire_front(bool wait)
    {
        const Region f = inflight_.front();
        int rc = wait ? ops_.wait(f.ev) : ops_.poll(f.ev);
        if (rc < 0)
            return rc;
        if (!wait && rc == 0)
            return 0;
        ops_.recycle(f.ev);
        inflight_.pop_front();
        if (inflight_.empty())
            head_ = 0;
        return 1;
    }

    Ops ops_;
    uint64_t cap_ = 0, head_ = 0;
    std::deque<Region> inflight_;
};

}  // namespace kvc
