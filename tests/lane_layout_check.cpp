// Host-side check of the kernels' direct-to-LDS tile loads, calling the
// same per-lane addressing functions the kernels call (lane_layout.h).
// For every wavefront of a workgroup, every lane and every load number:
//   * a real load reads 16 bytes inside its [64 x row] source tile and
//     writes 16 bytes inside its LDS slot; the real loads of a tile cover
//     every 16-byte chunk of the source tile (each data chunk of an LDS row
//     exactly once), so no LDS byte is left stale;
//   * a load without a number (uneven split) writes inside the 1 KB sink;
//   * the buffer resource a tile is read through lies inside the tensor's
//     (batch, head) sequence, and a lane's offset is in range only for rows
//     below the valid length, for every valid length and tile of the plan;
//   * 32-bit byte offsets stay below 2^32 up to the sequence length the
//     entry points accept (2^31 bytes for the whole-sequence resources).
// Prints one line per failure and exits with status 1 if any.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "lane_layout.h"

using namespace miattn::lanes;

static int g_fails = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      if (g_fails++ < 20) {                               \
        std::printf("FAIL line %d: ", __LINE__);          \
        std::printf(__VA_ARGS__);                         \
        std::printf("\n");                                \
      }                                                   \
    }                                                     \
  } while (0)

// Loads of one tile dealt to NW waves: (wave, m) -> load number w + NW m.
// src(i, lane) gives the source offset, row_bytes the source row size,
// lds_chunks the LDS chunks per row (data chunks first, then pads).
template <typename Src>
static void check_tile(const char* what, int NW, int nloads, int rows,
                       int row_bytes, int lds_chunks, Src src) {
  const int tile_bytes = rows * row_bytes;
  const int data_chunks = row_bytes / 16;
  const int slot_bytes = rows * lds_chunks * 16;
  std::vector<int> lds_written(rows * lds_chunks, 0);
  std::vector<int> src_read(rows * data_chunks, 0);
  const int per_wave = (nloads + NW - 1) / NW;
  for (int w = 0; w < NW; ++w)
    for (int m = 0; m < per_wave; ++m) {
      const int i = w + NW * m;
      for (int lane = 0; lane < 64; ++lane) {
        if (i >= nloads) {
          CHECK(lane * 16 + 16 <= 1024, "%s sink write", what);
          continue;
        }
        const unsigned s = src(i, lane);
        CHECK(s % 16 == 0 && s + 16 <= (unsigned)tile_bytes,
              "%s: load %d lane %d reads bytes %u..%u of a %d-byte tile",
              what, i, lane, s, s + 15, tile_bytes);
        const int dst = i * 1024 + lane * 16;
        CHECK(dst + 16 <= slot_bytes,
              "%s: load %d lane %d writes LDS bytes %d..%d of %d", what, i,
              lane, dst, dst + 15, slot_bytes);
        if (s + 16 > (unsigned)tile_bytes || dst + 16 > slot_bytes) continue;
        const int lrow = (dst / 16) / lds_chunks;
        const int lchunk = (dst / 16) % lds_chunks;
        lds_written[lrow * lds_chunks + lchunk]++;
        if (lchunk < data_chunks) src_read[s / 16]++;
      }
    }
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < lds_chunks; ++c)
      CHECK(lds_written[r * lds_chunks + c] == 1,
            "%s: LDS row %d chunk %d written %d times", what, r, c,
            lds_written[r * lds_chunks + c]);
  for (int k = 0; k < rows * data_chunks; ++k)
    CHECK(src_read[k] == 1, "%s: source chunk %d read %d times", what, k,
          src_read[k]);
}

// prefill: K rows in MFMA order, V rows in key order, padded LDS rows
static void check_prefill(int D) {
  char what[64];
  std::snprintf(what, sizeof(what), "prefill K d=%d", D);
  check_tile(what, kPrefillWaves, prefill_k_loads(D), kTileRows, D * 2,
             prefill_k_chunks(D), [&](int i, int lane) {
               return prefill_k_src(D, i, lane);
             });
  std::snprintf(what, sizeof(what), "prefill V d=%d", D);
  check_tile(what, kPrefillWaves, prefill_v_loads(D), kTileRows, D * 2,
             prefill_v_chunks(D), [&](int i, int lane) {
               return prefill_v_src(D, i, lane);
             });
  // per-tile resources: [tile, tile + bytes) inside the sequence, and an
  // in-range lane offset always names a row below the valid length
  const int Nks[] = {1, 17, 63, 64, 65, 300, 1024, 4097};
  for (int Nk : Nks) {
    const int nt = (Nk + kTileRows - 1) / kTileRows;
    const int Ls[] = {0, 1, Nk / 2, Nk - 1, Nk};
    for (int L : Ls) {
      if (L < 0) continue;
      for (int t = 0; t <= nt + 1; ++t)
        for (int live = 0; live < 2; ++live) {
          const int bytes = prefill_tile_bytes(D, L, t, live);
          const long long begin = (long long)t * kTileRows * D * 2;
          CHECK(bytes >= 0 && bytes <= kTileRows * D * 2,
                "prefill d=%d tile bytes %d", D, bytes);
          if (bytes > 0)
            CHECK(begin + bytes <= (long long)L * D * 2,
                  "prefill d=%d Nk=%d L=%d t=%d: resource ends at %lld past "
                  "the valid rows (%lld bytes)",
                  D, Nk, L, t, begin + bytes, (long long)L * D * 2);
          for (int i = 0; i < prefill_k_loads(D); ++i)
            for (int lane = 0; lane < 64; ++lane) {
              const unsigned s = prefill_k_src(D, i, lane);
              if (s < (unsigned)bytes)
                CHECK(t * kTileRows + (int)(s / (D * 2)) < L,
                      "prefill d=%d: key row past L read", D);
            }
        }
    }
  }
}

// backward: unpadded [64][D] tiles with the XOR chunk permutation, read
// through one resource per sequence with the tile's offset added per lane
static void check_bwd(int D) {
  char what[64];
  std::snprintf(what, sizeof(what), "backward tile d=%d", D);
  check_tile(what, kBwdWaves, bwd_tile_loads(D), kTileRows, D * 2, D / 8,
             [&](int i, int lane) { return bwd_tile_src(D, i, lane); });
  // the largest accepted sequence: rows * D * 2 < 2^31 bytes; the last
  // tile's largest lane offset must stay below 2^32
  const long long max_rows = ((1LL << 31) - 1) / (D * 2);
  const long long last_tile = (max_rows + kTileRows - 1) / kTileRows - 1;
  unsigned max_src = 0;
  for (int i = 0; i < bwd_tile_loads(D); ++i)
    for (int lane = 0; lane < 64; ++lane)
      if (bwd_tile_src(D, i, lane) > max_src) max_src = bwd_tile_src(D, i, lane);
  const long long top = last_tile * kTileRows * D * 2 + max_src + 16;
  CHECK(top < (1LL << 32), "backward d=%d: offset %lld overflows 32 bits", D,
        top);
  // in-range offsets name rows below the valid length
  const int Ls[] = {1, 63, 64, 65, 300, 4096};
  for (int L : Ls) {
    const long long bytes = (long long)L * D * 2;
    const int nt = (L + kTileRows - 1) / kTileRows + 1;
    for (int t = 0; t < nt; ++t)
      for (int i = 0; i < bwd_tile_loads(D); ++i)
        for (int lane = 0; lane < 64; ++lane) {
          const long long off =
              (long long)t * kTileRows * D * 2 + bwd_tile_src(D, i, lane);
          if (off < bytes)
            CHECK(off / (D * 2) < L, "backward d=%d: row past L read", D);
        }
  }
}

// FP8 forward: K codes [64][D] bytes, V^T codes [D][64] bytes, both read
// through one resource per (batch, K/V head) over whole 64-key tiles
static void check_fp8(int D) {
  char what[64];
  std::snprintf(what, sizeof(what), "fp8 K d=%d", D);
  check_tile(what, kFp8Waves, fp8_k_loads(D), kTileRows, D, D / 16,
             [&](int i, int lane) { return fp8_k_src(D, i, lane); });
  std::snprintf(what, sizeof(what), "fp8 V^T d=%d", D);
  check_tile(what, kFp8Waves, fp8_v_loads(D), D, 64, 4,
             [&](int i, int lane) { return fp8_v_src(i, lane); });
  const long long max_keys = ((1LL << 31) - 1) / (D * 2) / 64 * 64;
  const long long top = max_keys * D;  // bytes of the padded code sequence
  CHECK(top < (1LL << 32), "fp8 d=%d: code offsets overflow 32 bits", D);
}

int main() {
  for (int D : {64, 128}) {
    check_prefill(D);
    check_bwd(D);
    check_fp8(D);
  }
  if (g_fails) {
    std::printf("%d failures\n", g_fails);
    return 1;
  }
  std::printf("lane layout: all checks passed\n");
  return 0;
}
