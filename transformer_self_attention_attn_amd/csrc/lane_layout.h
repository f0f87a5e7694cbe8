// Per-lane addressing of the kernels' direct-to-LDS tile loads, and the byte
// ranges of the buffer resources they read through.  Plain integer
// arithmetic with no HIP dependency: the kernels call these functions on the
// device, and a host program in the test suite calls the same functions to
// check every lane's source offset, LDS destination and resource range
// without a GPU.  Internal; not installed.
//
// The loads: a wave-wide 16-byte direct-to-LDS load writes 1 KB of LDS,
// lane l the 16 bytes at destination + 16 l, and reads from the buffer
// resource at the lane's byte offset.  A tile of 64 rows is split into wave
// loads i = 0 .. n-1, dealt round-robin to the waves (wave w issues loads
// w, w + NW, ...); a wave with no load number left writes into a sink or
// skips the load.  A read at or past the resource's end returns zeros.
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define MIATTN_HD __host__ __device__
#else
#define MIATTN_HD
#endif

namespace miattn {
namespace lanes {

// Workgroup shapes (wavefronts) of the kernels that issue such loads.
constexpr int kPrefillWaves = 4;  // prefill_bf16.hip, d = 64 and 128
constexpr int kBwdWaves = 4;      // bwd_bf16.hip, dK/dV and dQ kernels
constexpr int kFp8Waves = 4;      // fp8.hip, forward kernel
constexpr int kTileRows = 64;     // rows (keys or queries) of a tile

// Row of a 32-row MFMA A-operand block that holds tile row m: with this
// order the 32x32 accumulator gives lane group g (lanes 32g .. 32g+31) the
// 16 consecutive tile rows 16g .. 16g+15 of each 32-row block.
MIATTN_HD constexpr int mfma_row(int m) {
  return (m >> 5) * 32 + ((m >> 2) & 1) * 16 + ((m & 31) >> 3) * 4 + (m & 3);
}

// ---- prefill (bf16, Nq > 1) ---------------------------------------------
// LDS tiles are padded: a K row is D + 8 elements (D/8 + 1 chunks of 16
// bytes), a V row D + 32 (D/8 + 4); pad chunks take the row's first chunk.
// K rows are stored in MFMA row order, V rows in key order.
MIATTN_HD constexpr int prefill_k_chunks(int D) { return D / 8 + 1; }
MIATTN_HD constexpr int prefill_v_chunks(int D) { return D / 8 + 4; }
MIATTN_HD constexpr int prefill_k_loads(int D) {
  return kTileRows * prefill_k_chunks(D) / 64;
}
MIATTN_HD constexpr int prefill_v_loads(int D) {
  return kTileRows * prefill_v_chunks(D) / 64;
}
// Byte offset within the source tile of lane `lane`'s part of load i.
// (row and chunk from unsigned division: a multiply-high and a shift on the
// device, where signed division by a constant needs sign fix-ups)
MIATTN_HD constexpr unsigned prefill_k_src(int D, int i, int lane) {
  const unsigned s = (unsigned)(i * 64 + lane);
  const unsigned n = (unsigned)prefill_k_chunks(D);
  const int r = (int)(s / n), c = (int)(s % n);
  return 2u * (unsigned)(mfma_row(r) * D + (c < D / 8 ? c * 8 : 0));
}
MIATTN_HD constexpr unsigned prefill_v_src(int D, int i, int lane) {
  const unsigned s = (unsigned)(i * 64 + lane);
  const unsigned n = (unsigned)prefill_v_chunks(D);
  const int r = (int)(s / n), c = (int)(s % n);
  return 2u * (unsigned)(r * D + (c < D / 8 ? c * 8 : 0));
}
// Bytes of tile t's resource: its rows below the valid length L (0 for a
// step past the plan), starting at the tile.
// (Written without a plain clamp, which the device compiler turns into a
// vector med3 and a readfirstlane; this form stays on the scalar unit.)
MIATTN_HD constexpr int prefill_tile_bytes(int D, int L, int t, bool live) {
  const int rem = L - t * kTileRows;  // rows of the sequence from the tile on
  const int over = rem > kTileRows ? rem - kTileRows : 0;
  const int rows = rem - over;        // min(rem, 64)
  return live && rows > 0 ? rows * D * 2 : 0;
}

// ---- backward (bf16) ------------------------------------------------------
// Tiles are [64][D] unpadded; logical 16-byte chunk c of row r sits at chunk
// c ^ bwd_swz(r), which keeps row-wise and transposing operand reads free
// of bank conflicts.
MIATTN_HD constexpr int bwd_swz(int D, int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 1) + 2 * ((r >> 4) & 1)
                  : 4 * ((r >> 1) & 1) + ((r >> 2) & 1) + 2 * ((r >> 4) & 1);
}
MIATTN_HD constexpr int bwd_tile_loads(int D) {
  return kTileRows * (D / 8) / 64;
}
// Byte offset within a [64][D] tile of lane `lane`'s part of load i: row
// s / (D/8), logical chunk (s % (D/8)) ^ swz(row), s = 64 i + lane.
MIATTN_HD constexpr unsigned bwd_tile_src(int D, int i, int lane) {
  const int s = i * 64 + lane, ch = D / 8;
  const int r = s / ch;
  const int c = (s - r * ch) ^ bwd_swz(D, r);
  return (unsigned)((r * D + c * 8) * 2);
}

// ---- FP8 forward -----------------------------------------------------------
// K codes as [64 keys][D] bytes with chunk c of row r at c ^ fp8_swz_k(r);
// V^T codes as [D][64 keys] with chunk c of row r at c ^ fp8_swz_v(r).
MIATTN_HD constexpr int fp8_swz_k(int D, int r) {
  return D == 128 ? 4 * ((r >> 1) & 1) + ((r >> 2) & 1) + 2 * ((r >> 4) & 1)
                  : ((r >> 2) & 1) + 2 * ((r >> 4) & 1);
}
MIATTN_HD constexpr int fp8_swz_v(int r) { return (r >> 2) & 3; }
MIATTN_HD constexpr int fp8_k_loads(int D) { return kTileRows * D / 1024; }
MIATTN_HD constexpr int fp8_v_loads(int D) { return kTileRows * D / 1024; }
MIATTN_HD constexpr unsigned fp8_k_src(int D, int i, int lane) {
  const int sl = i * 64 + lane;
  const int row = sl / (D / 16);
  const int c = (sl - row * (D / 16)) ^ fp8_swz_k(D, row);
  return (unsigned)(row * D + 16 * c);
}
MIATTN_HD constexpr unsigned fp8_v_src(int i, int lane) {
  const int sl = i * 64 + lane;
  const int row = sl / 4;
  const int c = (sl - row * 4) ^ fp8_swz_v(row);
  return (unsigned)(row * 64 + 16 * c);
}

}  // namespace lanes
}  // namespace miattn
