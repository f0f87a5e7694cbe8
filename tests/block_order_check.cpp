// Host check of block_order.h, the order in which the forward kernels deal
// their query blocks to the XCDs.  For each shape, over every block id:
//   * block_pos is a bijection onto (batch, K/V head, head, query block);
//   * it equals a reference written with plain integer division;
//   * on the longest-first path, every block of a (batch, K/V head) group
//     runs on one XCD (block id mod 8), and within a band the blocks of a
//     group come heaviest (highest query block) first, a band covering
//     qband consecutive query blocks.
// Prints one line per failure and exits with status 1 if any.
#include <cstdio>
#include <vector>

#include "block_order.h"
#include "tail_queue.h"

using namespace miattn;

static int g_fails = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      if (g_fails++ < 20) {                      \
        std::printf("FAIL line %d: ", __LINE__); \
        std::printf(__VA_ARGS__);                \
        std::printf("\n");                       \
      }                                          \
    }                                            \
  } while (0)

// the same order with plain division
static BlockPos reference(int bid, int B, int Hkv, int G, int nqb,
                          bool causal, int qband) {
  const int n = B * Hkv * G * nqb, ngrp = B * Hkv;
  const int xcd = bid % 8, slot = bid / 8;
  int grp, qrank, hh;
  if (causal && ngrp % 8 == 0) {
    const int gpx = ngrp / 8, bs = qband * G;
    const int band = slot / (gpx * bs);
    const int r1 = slot % (gpx * bs);
    const int gi = r1 / bs, r2 = r1 % bs;
    qrank = band * qband + r2 / G;
    grp = xcd * gpx + gi;
    hh = r2 % G;
  } else {
    const int per = n / 8, rem = n % 8;
    const int lid = xcd * per + (xcd < rem ? xcd : rem) + slot;
    grp = lid / (G * nqb);
    qrank = (lid % (G * nqb)) / G;
    hh = lid % G;
  }
  BlockPos p;
  p.qb = causal ? nqb - 1 - qrank : qrank;
  p.b = grp / Hkv;
  p.hk = grp % Hkv;
  p.hh = hh;
  return p;
}

static void check_shape(int B, int Hkv, int G, int nqb, bool causal,
                        long long kvb, int slots) {
  const BlockOrder o = make_block_order(B, Hkv, G, nqb, causal, kvb, slots);
  const int n = o.total;
  CHECK(n == B * Hkv * G * nqb, "total");
  std::vector<int> seen(n, 0);
  std::vector<int> grp_xcd(B * Hkv, -1);
  std::vector<int> last_qb(8 * B * Hkv * (nqb + 1), 1 << 30);
  for (int bid = 0; bid < n; ++bid) {
    const BlockPos p = block_pos(bid, o);
    const bool in = p.b >= 0 && p.b < B && p.hk >= 0 && p.hk < Hkv &&
                    p.hh >= 0 && p.hh < G && p.qb >= 0 && p.qb < nqb;
    CHECK(in, "B%d Hkv%d G%d nqb%d: bid %d maps out of range", B, Hkv, G, nqb,
          bid);
    if (!in) continue;
    const int key = ((p.b * Hkv + p.hk) * G + p.hh) * nqb + p.qb;
    seen[key]++;
    const BlockPos r = reference(bid, B, Hkv, G, nqb, causal, o.qband);
    CHECK(r.b == p.b && r.hk == p.hk && r.hh == p.hh && r.qb == p.qb,
          "B%d Hkv%d G%d nqb%d: bid %d differs from the reference", B, Hkv, G,
          nqb, bid);
    if (o.lpt) {
      const int grp = p.b * Hkv + p.hk, xcd = bid % 8;
      if (grp_xcd[grp] < 0) grp_xcd[grp] = xcd;
      CHECK(grp_xcd[grp] == xcd, "group %d on two XCDs", grp);
      const int slot = bid / 8;
      const int band = slot / (o.gpx * o.qband * G);
      CHECK(nqb - 1 - p.qb >= band * o.qband &&
                nqb - 1 - p.qb < (band + 1) * o.qband,
            "bid %d: query block %d outside band %d", bid, p.qb, band);
      int& lq = last_qb[(xcd * B * Hkv + grp) * (nqb + 1) + band];
      CHECK(p.qb <= lq, "bid %d: lighter block before a heavier one", bid);
      lq = p.qb;
    }
  }
  for (int k = 0; k < n; ++k)
    CHECK(seen[k] == 1, "B%d Hkv%d G%d nqb%d: block %d seen %d times", B, Hkv,
          G, nqb, k, seen[k]);
}

// The run-time tail of tail_queue.h: the fixed blocks (ids below first, the
// first three quarters of every XCD's list) and the blocks of tickets
// 0 .. ndyn-1 (id first + ticket while below total) cover every block once,
// with enough dynamic workgroups for the whole tail; off, the grid is the
// block count.
static void check_tail(int total, int slots, bool on, bool expect_on) {
  int grid = -1;
  const TailQueue q = make_tail_queue(total, slots, 3, on, &grid);
  if (!expect_on) {
    CHECK(q.first == total && q.ndyn == 0 && grid == total,
          "tail total=%d: expected off, first=%d ndyn=%d grid=%d", total,
          q.first, q.ndyn, grid);
    return;
  }
  CHECK(q.first % kTailXcds == 0 && q.first < total,
        "tail total=%d: first=%d", total, q.first);
  CHECK(q.first / kTailXcds == total / kTailXcds - total / kTailXcds / 4,
        "tail total=%d: split slot %d", total, q.first / kTailXcds);
  CHECK(grid >= total && q.ndyn == grid - q.first && q.ndyn >= total - q.first,
        "tail total=%d: grid=%d ndyn=%d", total, grid, q.ndyn);
  CHECK(q.set >= 0 && q.set < kTailSets, "tail set %d", q.set);
  std::vector<int> seen(total, 0);
  for (int b = 0; b < q.first; ++b) seen[b]++;
  for (int t = 0; t < q.ndyn; ++t)
    if (q.first + t < total) seen[q.first + t]++;
  for (int b = 0; b < total; ++b)
    CHECK(seen[b] == 1, "tail total=%d: block %d run %d times", total, b,
          seen[b]);
}

int main() {
  check_shape(4, 4, 7, 32, true, 2LL << 20, 64);     // gqa-causal-prefill
  check_shape(16, 12, 1, 8, true, 256LL << 10, 96);  // gpt2-small-causal-padded
  check_shape(2, 16, 1, 128, true, 4LL << 20, 96);   // sliding-window-causal
  check_shape(3, 5, 3, 7, true, 4LL << 20, 64);      // groups not divisible by 8
  check_shape(2, 4, 4, 10, false, 4LL << 20, 64);    // no causal mask
  check_shape(8, 8, 16, 64, true, 4LL << 20, 64);    // bands of several blocks
  check_shape(1, 1, 1, 1, true, 1024, 64);           // one block
  check_tail(4 * 4 * 7 * 32, 64, true, true);    // gqa-causal-prefill
  check_tail(8 * 8 * 16 * 64, 64, true, true);   // many blocks
  check_tail(3 * 8 * 64 + 5, 64, true, true);    // not a multiple of 8
  check_tail(16 * 12 * 8, 96, true, false);      // under three rounds
  check_tail(2 * 16 * 128, 96, false, false);    // not asked for
  if (g_fails) {
    std::printf("%d failures\n", g_fails);
    return 1;
  }
  std::printf("block order: all checks passed\n");
  return 0;
}
