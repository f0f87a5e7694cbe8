// A run-time queue for the light tail of a causal launch.
// Internal; not installed.
//
// The hardware deals workgroups to the 8 XCDs round-robin, a fixed share
// each (block_order.h), but the XCDs of one chip do not run equally fast:
// under a long matrix-core load their loop steps differ by several percent,
// and with fixed shares the fast XCDs idle at the end while the slow ones
// finish.  Under the causal mask the longest-first order leaves the lightest
// blocks at the end of every XCD's list, so the last quarter of each list is
// handed out at run time instead: the workgroups from a split point on take
// tickets from one device-wide counter, ticket t running block first + t
// (the XCDs' tails interleaved, still heaviest first), and the launch has a
// quarter of that tail in spare workgroups, so an XCD that runs ahead takes
// more of the tail.  A workgroup that finds the tail empty exits at once.
// Light blocks read few K/V tiles, so running one away from its group's
// XCD costs little; tails of uniform blocks (a left window) stay fixed,
// since their K/V is then fetched by several L2s.
//
// Counters: sets of 16 words in a file-scope device array (zero when the
// code object loads): word 0 counts tickets, word 1 the dynamic workgroups
// that took theirs.  Each launch takes the next set of a ring of 64 on the
// host (a captured graph keeps the set of its capture); the launch's last
// workgroup to take a ticket zeroes the set, so it is clean when the launch
// ends.  Launches that overlap in time on one device and hold the same set
// would race.
#pragma once

#include <atomic>

namespace miattn {

constexpr int kTailSets = 64;
constexpr int kTailXcds = 8;

struct TailQueue {
  int first;  // block id of the first dynamic workgroup (total when off)
  int ndyn;   // dynamic workgroups in the launch (grid - first); 0 when off
  int set;    // counter set of this launch
};

// The queue of a launch of `total` blocks; *grid receives the launch's
// workgroup count.  Off (grid = total) unless `on` and the launch fills the
// chip's slots min_rounds times or more.
inline TailQueue make_tail_queue(int total, int slots_per_xcd, int min_rounds,
                                 bool on, int* grid) {
  static std::atomic<unsigned> next_set{0};
  TailQueue q{total, 0, 0};
  *grid = total;
  const int n_min = total / kTailXcds;  // blocks of the shortest list
  const int dyn = n_min / 4;            // tail blocks per XCD
  if (!on || total < min_rounds * kTailXcds * slots_per_xcd || dyn < 4)
    return q;
  q.first = kTailXcds * (n_min - dyn);
  *grid = total + kTailXcds * (dyn / 4);
  q.ndyn = *grid - q.first;
  q.set = (int)(next_set.fetch_add(1u, std::memory_order_relaxed) % kTailSets);
  return q;
}

#if defined(__HIPCC__)
namespace {
__device__ unsigned g_tail_counters[kTailSets * 16];
}

// Taken by one thread of a dynamic workgroup: the block id it runs, or -1
// when the tail is empty.  *done receives the count of dynamic workgroups
// that took their ticket before this one (passed on to tail_clear).
__device__ inline int tail_take(const TailQueue& q, int total,
                                unsigned* done) {
  unsigned* c = g_tail_counters + 16 * q.set;
  const unsigned t = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  // the count below is issued only once the ticket has returned, so the
  // launch's last count follows every one of its tickets
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  *done = __hip_atomic_fetch_add(c + 1, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  return q.first + (int)t < total ? q.first + (int)t : -1;
}

// Zeroes the set when `done` marks the launch's last ticket taker: every
// dynamic workgroup has then taken its ticket.
__device__ inline void tail_clear(const TailQueue& q, unsigned done) {
  if (done + 1 != (unsigned)q.ndyn) return;
  unsigned* c = g_tail_counters + 16 * q.set;
  __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(c + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
#endif

}  // namespace miattn
