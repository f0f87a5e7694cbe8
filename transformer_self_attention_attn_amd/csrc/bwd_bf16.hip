// Backward pass of bf16 attention on gfx950 matrix cores: dQ, dK and dV of
// O = softmax(scale * Q K^T + mask) V given dO, the forward output O and its
// log-sum-exp.  The FlashAttention-3 review page names this pass (dQ, dK, dV;
// about 2.5 times the forward FLOPs) without printing its equations; what is
// computed is the exact gradient of the forward function, by the chain rule
// through its steps:
//   p_ij  = exp(scale * q_i . k_j - lse_i)         (allowed pairs, else 0)
//   dV_j  = sum_i p_ij dO_i
//   dp_ij = dO_i . v_j
//   ds_ij = p_ij (dp_ij - delta_i),   delta_i = sum_j p_ij dp_ij = dO_i . O_i
//   dQ_i  = scale * sum_j ds_ij k_j,  dK_j = scale * sum_i ds_ij q_i
// with K/V gradients summed over the query heads of a group, and zero for
// padding keys, dead rows and masked pairs.  The mask (causal, valid length,
// two-sided window, sink keys) and the row positions are those of the forward
// kernels.
//
// Three launches, no atomics (results do not depend on scheduling):
//   bwd_pre   -delta_i from dO and O, and lse_i * log2(e), per query row,
//             into a workspace padded to 64 rows; a row that sees no key gets
//             +inf, so every probability of it is exactly 0.
//   bwd_dkdv  one workgroup per (batch, K/V head, block of 32*NW keys); wave
//             w owns 32 keys and holds their K and V as MFMA B operands in
//             registers; the workgroup streams 64-row tiles of Q and dO (with
//             their lse and delta) of every query head of the group through
//             LDS, and each wave forms
//               S  = Q K^T   and  dP = dO V^T   (A = Q / dO rows from LDS)
//               P, dS in registers (lane = key, 16 consecutive queries)
//               dV^T += dO^T P   and  dK^T += Q^T dS   (A = transposing LDS
//                                                      reads of dO / Q)
//   bwd_dq    one workgroup per (batch, query head, block of 32*NW rows),
//             shaped like the forward kernel: wave w owns 32 rows and holds
//             their Q and dO as B operands; 64-key tiles of K and V stream
//             through LDS and each wave forms
//               S^T = K Q^T  and  dP^T = V dO^T
//               dS^T in registers (lane = query, 16 consecutive keys)
//               dQ^T += K^T dS^T   (A = transposing LDS reads of K)
// Tiles arrive by 16-byte direct-to-LDS buffer loads into ring slots (three
// in bwd_dkdv, two in bwd_dq), each slot its own LDS object named by a
// compile-time index; rows past the valid length (or dead query rows) lie
// outside the buffer resource and read zeros, so padded contents never enter
// a product.  A tile is read two ways: row-wise (16
// bytes per lane, the A operand of Q K^T) and column-wise (the transposing
// read, the A operand of dO^T P); tiles are stored unpadded with the 16-byte
// chunks of each row permuted by an XOR of row bits (see swz), which keeps
// both kinds of read free of LDS bank conflicts.
// The dK/dV step reads its MFMA operands from a ring four MFMAs ahead.  At
// d=64 the step is one sequence of MFMAs in which the softmax of one 32-row
// half of the tile runs between the MFMAs of the other half; at d=128 the
// halves pass through a three-stream pipeline (products of the next half,
// softmax of this one, gradient products of the previous one), so that the
// exponentials spread over every MFMA of the step.  In both gradient kernels
// the steps whose tiles every row (or key) of the wave fully sees run in a
// loop of their own, with no mask construction or per-step test; bwd_dq
// deals its blocks in the forward kernels' order (block_order.h).
#include "kernels.h"

#include <cmath>
#include <type_traits>

#include "block_order.h"
#include "device_common.h"


namespace miattn {
namespace bwd_impl {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kRT = 64;    // rows of a streamed tile (queries or keys)
constexpr int kWR = 32;    // rows a wave owns (keys in dK/dV, queries in dQ)

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* lse2;   // [B*Hq][Nqp]: lse * log2(e); +inf on rows that see no key
  float* delta;  // [B*Hq][Nqp]: -(dO . O); 0 on those rows
  const int* seqlens;
  int B, Hq, Hkv, Nq, Nk, Nqp, G, causal, window, window_right, sinks;
  int nblk, total;  // blocks per (batch, head) and in the grid
  float c;          // scale * log2(e)
  float scale;
  BlockOrder order;  // dQ kernel: block -> (batch, head, query block)
};

template <int D>
struct BCfg {
  static constexpr int CH = D / 8;            // 16-byte chunks per tile row
  static constexpr int TILE = kRT * D;        // elements per tile (unpadded)
  static constexpr int LOADS = kRT * CH / 64; // wave-wide 1 KB loads per tile
  static constexpr int KS = D / 16;           // k-steps of a D-long product
  static constexpr int DB = D / 32;           // 32-row blocks of a D^T result
  static_assert(kRT * CH % 64 == 0, "tile loads");
};

// Chunk permutation of a tile row: logical 16-byte chunk c of row r sits at
// chunk c ^ swz(r).  A row-wise operand read has 16 lanes read one chunk of
// 16 different rows (rows mfma_row(0..15) and the like), a transposing read
// has 32 lanes read chunks 4m .. 4m+3 of 4 consecutive rows; with this XOR
// each such group covers the 64 four-byte LDS banks once (d=128: one row per
// 256-byte bank line; d=64: two).
template <int D>
__device__ inline int swz(int r) {
  return lanes::bwd_swz(D, r);
}

// One wave-wide direct-to-LDS load of a [64][D] tile: wave load i fills
// tile bytes [i*1024, +1024); lane l writes 16-byte slot s = i*64 + l, which
// is physical chunk s % CH of row s / CH and so holds that row's logical
// chunk (s % CH) ^ swz(row).  Loads go through a buffer resource whose size
// ends at the last valid row, with the whole offset in the per-lane operand,
// so a row past the valid length reads zeros.
// Byte offset, within a [64][D] tile, of the source of this lane's part of
// wave load i: row s / CH, logical chunk (s % CH) ^ swz(row).
template <int D>
__device__ inline unsigned tile_src_off(int i, int lane) {
  static_assert(BCfg<D>::LOADS == lanes::bwd_tile_loads(D), "tile loads");
  return lanes::bwd_tile_src(D, i, lane);
}

// Element offset of this lane's row-wise A-operand piece: tile row
// mfma_row(32 mb + lane % 32), columns 16 ks + 8 g .. +7 (g = lane / 32).
template <int D>
__device__ inline int a_off(int lane, int mb, int ks) {
  const int row = mfma_row(mb * 32 + (lane & 31));
  return row * D + 8 * ((2 * ks + (lane >> 5)) ^ swz<D>(row));
}

// Element offset of this lane's 8-byte piece of a transposing read of tile
// rows R .. R+3, R = 32 mb + 16 g + 8 m2 + 4 half, columns 32 db .. +31,
// less the part (32 mb + 8 m2 + 4 half) * D that is a compile-time constant
// at every use.  Lane i of each 16-lane group addresses row R + i / 4,
// columns 32 db + 16 (lane / 16 % 2) + 4 (i % 4) .. +3; with R % 4 == 0 the
// chunk permutation of that row is fj + half + 2 g.
template <int D>
__device__ inline int tr_off(int lane, int half, int db) {
  const int g = lane >> 5, grp16 = lane >> 4, i16 = lane & 15;
  const int j = i16 >> 2;
  const int fj = (D == 128) ? 4 * j : 4 * ((j >> 1) & 1);
  const int lb = 2 * (grp16 & 1) + ((i16 & 3) >> 1);
  const int pc = 4 * (db ^ (fj >> 2)) + (lb ^ (half + 2 * g));
  return (16 * g + j) * D + 8 * pc + 4 * (i16 & 1);
}

// A operand of X^T for the lane's k-group: rows R .. R+7 (two transposing
// reads of four rows), columns 32 db .. +31; off = tr_off(lane, 0/1, db).
__device__ inline bf16x8 tr_pair(const uint16_t* p0, const uint16_t* p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = __builtin_bit_cast(__bf16, (short)a[e]);
    r[4 + e] = __builtin_bit_cast(__bf16, (short)b[e]);
  }
  return r;
}

// ---------------------------------------------------------------------------
// bwd_pre: one 64-lane wave covers 64*8/D rows; D/8 lanes per row.

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long row = gw * RPW + lane / LPR;  // over B*Hq*Nqp
  const long long total = (long long)p.B * p.Hq * p.Nqp;
  const bool valid = row < total;
  const int bh = valid ? (int)(row / p.Nqp) : 0;
  const int i = valid ? (int)(row - (long long)bh * p.Nqp) : 0;
  const Seq s = seq_of(p.seqlens, p.Nq, p.Nk, bh / p.Hq);
  float lse = -INFINITY;
  if (valid && i < s.Lq) lse = p.lse[(size_t)bh * p.Nq + i];
  const bool live = valid && i < s.Lq && lse > -INFINITY;
  float acc = 0.f;
  if (live) {
    const size_t off = ((size_t)bh * p.Nq + i) * D + (lane % LPR) * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(p.dout + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p.o + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16),
                 acc);
      acc = fmaf(__uint_as_float(a[e] & 0xffff0000u),
                 __uint_as_float(b[e] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int x = 1; x < LPR; x <<= 1) acc += __shfl_xor(acc, x);
  if (valid && lane % LPR == 0) {
    p.delta[row] = live ? -acc : 0.f;
    p.lse2[row] = live ? lse * 1.4426950408889634f : INFINITY;
  }
}

// ---------------------------------------------------------------------------
// bwd_dkdv

// PIPE: the step runs as the three-stream pipeline described below (d=128);
// otherwise as one sequence of MFMAs per tile (d=64, whose workgroups walk
// few tiles: the pipeline's fill and drain and the fully masked tiles it
// computes cost more there than it gains).
template <int D, int NW, bool PIPE>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dkdv_kernel(
    BwdParams p) {
  using C = BCfg<D>;
  constexpr int KB = kWR * NW;  // keys per workgroup
  // three ring slots of (Q tile, dO tile, lse, delta)
  __shared__ __attribute__((aligned(16))) uint16_t Qs0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Qs1[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Qs2[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Os0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Os1[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Os2[C::TILE];
  __shared__ __attribute__((aligned(16))) float Ls0[kRT];
  __shared__ __attribute__((aligned(16))) float Ls1[kRT];
  __shared__ __attribute__((aligned(16))) float Ls2[kRT];
  __shared__ __attribute__((aligned(16))) float Ds0[kRT];
  __shared__ __attribute__((aligned(16))) float Ds1[kRT];
  __shared__ __attribute__((aligned(16))) float Ds2[kRT];
  auto qslot = [&](auto s) -> uint16_t* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return Qs0; else if constexpr (S == 1) return Qs1;
    else return Qs2;
  };
  auto oslot = [&](auto s) -> uint16_t* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return Os0; else if constexpr (S == 1) return Os1;
    else return Os2;
  };
  auto lslot = [&](auto s) -> float* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return Ls0; else if constexpr (S == 1) return Ls1;
    else return Ls2;
  };
  auto dslot = [&](auto s) -> float* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return Ds0; else if constexpr (S == 1) return Ds1;
    else return Ds2;
  };

  // (batch, K/V head, key block), key blocks of one group adjacent; within a
  // group the low key blocks (more query rows under the causal mask) first
  const int lid = xcd_block(blockIdx.x, p.total);
  const int grp = lid / p.nblk;
  const int kb = lid - grp * p.nblk;
  const int b = grp / p.Hkv;
  const int hk = grp - b * p.Hkv;
  const Seq s = seq_of(p.seqlens, p.Nq, p.Nk, b);
  auto key_rows = [&](int key, int& lo, int& hi) {
    rows_of_key(s, p.causal, p.window, p.window_right, p.sinks, key, lo, hi);
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int kl = lane & 31;
  const int g = lane >> 5;
  const int k0 = kb * KB;
  const int kw0 = k0 + wave * kWR;
  const int j = kw0 + kl;  // this lane's key

  // rows that may see this lane's key, and over the wave: their hull (a tile
  // outside it is skipped) and their intersection (a tile inside it needs no
  // mask)
  int rlo, rhi;
  key_rows(j, rlo, rhi);
  const bool kne = rlo < rhi;
  // (wave-uniform; the pipelined step reads them back as scalars, so that
  // its tests are scalar branches)
  auto uni = [](int x) { return PIPE ? __builtin_amdgcn_readfirstlane(x) : x; };
  const int w_lo_min = uni(wave_imin(kne ? rlo : kBig));
  const int w_hi_max = uni(wave_imax(kne ? rhi : -kBig));
  const int w_lo_max = uni(wave_imax(rlo));
  const int w_hi_min = uni(wave_imin(rhi));
  // the workgroup's hull: the lowest key's first row and, unless the block
  // holds a sink key, the last valid key's end row
  int t0 = 0, nt = 0;
  if (k0 < s.L) {
    const int k1 = min(k0 + KB, s.L);
    int a_lo, a_hi, b_lo, b_hi;
    key_rows(k0, a_lo, a_hi);
    key_rows(k1 - 1, b_lo, b_hi);
    const int hi = k0 < p.sinks ? s.Lq : max(a_hi, b_hi);
    if (hi > a_lo) {
      t0 = a_lo / kRT;
      nt = (hi + kRT - 1) / kRT - t0;
    }
  }
  // (tile, query head) pairs, tile-major from the last tile down: every key
  // block of a group starts at the same tile and walks the same tiles in the
  // same order, so the blocks running together share each tile in L2
  const int nsteps = nt * p.G;
  const int t_last = t0 + nt - 1;
  auto wave_needs = [&](int t) {
    const int r0 = t * kRT;
    return r0 < w_hi_max && r0 + kRT > w_lo_min;
  };
  auto tile_full = [&](int t) {
    const int r0 = t * kRT;
    return r0 >= w_lo_max && r0 + kRT <= w_hi_min;
  };

  // K and V of this lane's key as B operands (8 consecutive columns per
  // k-step), zero past the valid length
  const size_t kv_base = (size_t)(b * p.Hkv + hk) * p.Nk * D;
  // The pipelined step forms S c with c > 0 (its mask relies on
  // -inf c = -inf): for a negative scale K is negated on load (its only use
  // is S) and c flipped; scale 0 takes a tiny positive c, under which every
  // allowed pair weighs the same.  The other step masks explicitly and
  // takes c as it is.
  const bool kneg = PIPE && p.c < 0.f;
  const float cc = !PIPE ? p.c : kneg ? -p.c : (p.c > 0.f ? p.c : 1e-30f);
  const unsigned ksign = kneg ? 0x80008000u : 0u;
  bf16x8 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 rk = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
    if (j < s.L) {
      rk = *reinterpret_cast<const u32x4*>(p.k + kv_base + (size_t)j * D +
                                           16 * ks + 8 * g);
      rv = *reinterpret_cast<const u32x4*>(p.v + kv_base + (size_t)j * D +
                                           16 * ks + 8 * g);
    }
    rk ^= ksign;
    kf[ks] = __builtin_bit_cast(bf16x8, rk);
    vf[ks] = __builtin_bit_cast(bf16x8, rv);
  }

  f32x16 dka[C::DB], dva[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dka[db][r] = 0.f;
      dva[db][r] = 0.f;
    }

  // lane offsets of the LDS operand reads (the same for the Q and dO tiles)
  int aoff[2][C::KS];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) aoff[mb][ks] = a_off<D>(lane, mb, ks);
  int toff[2][C::DB];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      toff[half][db] = tr_off<D>(lane, half, db);

  // loads of step u (query head hk*G + u % G, tile t_last - u / G) into
  // slot S.  A tile takes LOADS wave-wide loads, dealt round-robin: wave w
  // issues loads w, w + NW, ... (LOADS is a multiple of NW, so every wave
  // issues LOADS / NW of the Q tile and as many of the dO tile, at the same
  // per-lane offsets); waves 0 and 1 also load the tile's lse and delta (64
  // floats each).  Each load's kind is fixed at compile time.
  static_assert(C::LOADS % NW == 0 && NW >= 2, "loads per wave");
  constexpr int TW = C::LOADS / NW;  // tile loads per wave and tile
  constexpr int NL = 2 * C::LOADS + 2;
  unsigned toffs[TW];
#pragma unroll
  for (int m = 0; m < TW; ++m) toffs[m] = tile_src_off<D>(wave + NW * m, lane);
  const int qbytes = s.Lq * D * 2;  // rows past the live rows read zeros
  auto issue = [&](auto slot_c, int u) {
    const int h = hk * p.G + u % p.G;
    const int t = t_last - u / p.G;
    const int r0 = t * kRT;
    const size_t bh = (size_t)b * p.Hq + h;
    const auto qrs = rows_rsrc(p.q + bh * p.Nq * D, qbytes);
    const auto ors = rows_rsrc(p.dout + bh * p.Nq * D, qbytes);
    const int tb = r0 * D * 2;
#pragma unroll
    for (int m = 0; m < TW; ++m)
      miattn_buffer_load_lds(
          qrs, (lds_void*)(qslot(slot_c) + (wave + NW * m) * 512), 16,
          toffs[m] + tb, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < TW; ++m)
      miattn_buffer_load_lds(
          ors, (lds_void*)(oslot(slot_c) + (wave + NW * m) * 512), 16,
          toffs[m] + tb, 0, 0, 0);
    if (wave < 2) {
      const bool isl = wave == 0;
      const auto rs =
          rows_rsrc((isl ? p.lse2 : p.delta) + bh * p.Nqp, p.Nqp * 4);
      miattn_buffer_load_lds(
          rs, (lds_void*)(isl ? lslot(slot_c) : dslot(slot_c)), 4,
          (unsigned)(lane * 4) + r0 * 4, 0, 0, 0);
    }
  };

  if constexpr (!PIPE) {
    // One step, as a sequence of NM MFMAs:
    //   [0, NA)         S = Q K^T and dP = dO V^T of tile rows 0 .. 31
    //   [NA, 2NA)       the same for rows 32 .. 63, with P and dS of rows
    //                   0 .. 31 computed in between
    //   [2NA, 2NA+NB)   dV^T += dO^T P and dK^T += Q^T dS over rows 0 .. 31,
    //                   with P and dS of rows 32 .. 63 in between
    //   [2NA+NB, NM)    the same over rows 32 .. 63
    // Each MFMA's A operand is read from LDS four MFMAs ahead.
    constexpr int NA = 2 * C::KS;
    constexpr int NB = 4 * C::DB;
    constexpr int NM = 2 * NA + 2 * NB;
    constexpr int AHEAD = 4;
    constexpr int RING = AHEAD + 1;
    constexpr int EPS = 16 / NA;  // softmax elements per MFMA slot
    static_assert(NA == NB && 16 % NA == 0, "slots");

    // FULL: every (row, key) pair of the tile is allowed, no mask arithmetic
    auto compute_t = [&](auto slot_c, auto full_c, int t) {
      constexpr bool FULL = decltype(full_c)::value;
      const uint16_t* Qt = qslot(slot_c);
      const uint16_t* Ot = oslot(slot_c);
      const float* Lt = lslot(slot_c);
      const float* Dt = dslot(slot_c);

      auto fetch = [&](auto i_c) -> bf16x8 {
        constexpr int i = decltype(i_c)::value;
        if constexpr (i < 2 * NA) {
          constexpr int mb = i / NA, ks = (i % NA) / 2;
          const uint16_t* tb = (i % 2 == 0) ? Qt : Ot;
          return *reinterpret_cast<const bf16x8*>(tb + aoff[mb][ks]);
        } else {
          constexpr int x = i - 2 * NA;
          constexpr int mb = x / NB, r = x % NB;
          constexpr int m2 = r / (2 * C::DB), db = (r % (2 * C::DB)) / 2;
          const uint16_t* tb = (r % 2 == 0) ? Ot : Qt;
          constexpr int c0 = (32 * mb + 8 * m2) * D;
          return tr_pair(tb + toff[0][db] + c0, tb + toff[1][db] + c0 + 4 * D);
        }
      };

      f32x16 sa[2], pa[2];
      bf16x8 pb[2][2], sb[2][2];
      const f32x16 zero = {};
      // dP starts from -delta of its rows, so the accumulator ends at
      // dP - delta (the factor of dS besides P)
      f32x16 nd0[2];
  #pragma unroll
      for (int mb = 0; mb < 2; ++mb)
  #pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 d4 =
              *reinterpret_cast<const f32x4*>(Dt + mb * 32 + 16 * g + 4 * q4);
  #pragma unroll
          for (int e = 0; e < 4; ++e) nd0[mb][4 * q4 + e] = d4[e];
        }
      auto mfma = [&](auto i_c, const bf16x8& a) {
        constexpr int i = decltype(i_c)::value;
        if constexpr (i < 2 * NA) {
          constexpr int mb = i / NA, ks = (i % NA) / 2;
          if constexpr (i % 2 == 0)
            sa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, kf[ks], ks == 0 ? zero : sa[mb], 0, 0, 0);
          else
            pa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, vf[ks], ks == 0 ? nd0[mb] : pa[mb], 0, 0, 0);
        } else {
          constexpr int x = i - 2 * NA;
          constexpr int mb = x / NB, r = x % NB;
          constexpr int m2 = r / (2 * C::DB), db = (r % (2 * C::DB)) / 2;
          if constexpr (r % 2 == 0)
            dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[mb][m2],
                                                              dva[db], 0, 0, 0);
          else
            dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[mb][m2],
                                                              dka[db], 0, 0, 0);
        }
      };

      // softmax of rows 32 mb + 16 g + r of this tile (lane = key): a row
      // outside [rlo, rhi) is masked unless the tile is full
      const int r0 = t * kRT;
      float pvv[16], dsv[16];
      f32x4 l4;
      int mlo[2], mhi[2];
  #pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int base = r0 + mb * 32 + 16 * g;
        mlo[mb] = rlo - base;
        mhi[mb] = rhi - base;
      }
      auto element = [&](auto mb_c, auto r_c) {
        constexpr int mb = decltype(mb_c)::value, r = decltype(r_c)::value;
        if constexpr (r % 4 == 0)
          l4 = *reinterpret_cast<const f32x4*>(Lt + mb * 32 + 16 * g + r);
        float pr = __builtin_amdgcn_exp2f(fmaf(sa[mb][r], cc, -l4[r % 4]));
        if constexpr (!FULL) pr = (r >= mlo[mb] && r < mhi[mb]) ? pr : 0.f;
        pvv[r] = pr;
        dsv[r] = pr * pa[mb][r];
        if constexpr (r % 8 == 7) {
          constexpr int m2 = r / 8;
          f32x8 x, y;
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[e] = pvv[8 * m2 + e];
            y[e] = dsv[8 * m2 + e];
          }
          pb[mb][m2] = __builtin_convertvector(x, bf16x8);
          sb[mb][m2] = __builtin_convertvector(y, bf16x8);
        }
      };

      bf16x8 ring[RING];
      static_for<0, AHEAD>([&](auto i_c) {
        ring[decltype(i_c)::value] = fetch(i_c);
      });
      static_for<0, NM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        if constexpr (i + AHEAD < NM)
          ring[(i + AHEAD) % RING] = fetch(ic<i + AHEAD>());
        mfma(i_c, ring[i % RING]);
        // softmax of rows 0 .. 31 during slots [NA, 2NA), of rows 32 .. 63
        // during [2NA, 2NA+NB)
        if constexpr (i >= NA && i < 2 * NA + NB) {
          constexpr int mbs = (i < 2 * NA) ? 0 : 1;
          constexpr int k = (i < 2 * NA) ? i - NA : i - 2 * NA;
          static_for<0, EPS>([&](auto e_c) {
            element(ic<mbs>(), ic<k * EPS + decltype(e_c)::value>());
          });
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
      });
    };
    auto compute = [&](auto slot_c, int u) {
      const int t = t_last - u / p.G;
      if (!wave_needs(t)) return;
      if (tile_full(t))
        compute_t(slot_c, std::true_type(), t);
      else
        compute_t(slot_c, std::false_type(), t);
    };


    // step u computes from slot u % 3 while the loads of step u + 2 fill slot
    // (u + 2) % 3; before the barrier that ends step u each wave waits for its
    // loads of step u + 1 (all but the nl loads it issued for step u + 2)
    const int nl = (NL - wave + NW - 1) / NW;  // loads per step of this wave
    if (nsteps > 0) {
      issue(ic<0>(), 0);
      if (1 < nsteps) {
        issue(ic<1>(), 1);
        wait_vmcnt_rt(nl);
      } else {
        wait_vm0();
      }
      barrier_nofence();
      auto step = [&](auto slot_c, int u) {
        constexpr int S = decltype(slot_c)::value;
        const bool more = u + 2 < nsteps;
        if (more) issue(ic<(S + 2) % 3>(), u + 2);
        compute(slot_c, u);
        if (more)
          wait_vmcnt_rt(nl);
        else
          wait_vm0();
        barrier_nofence();
      };
      for (int u = 0; u < nsteps; u += 3) {
        step(ic<0>(), u);
        if (u + 1 < nsteps) step(ic<1>(), u + 1);
        if (u + 2 < nsteps) step(ic<2>(), u + 2);
      }
    }
  } else {
    // The work of a step is cut into two halves of 32 tile rows; half
    // H = 2u + m is rows 32m .. 32m+31 of step u's tile (slot u % 3).  Each
    // half passes through three stages:
    //   SdP(H)   S = Q K^T and dP = dO V^T - delta (NA MFMAs, A = row-wise
    //            LDS reads of Q / dO); on a tile that needs the mask, S starts
    //            from -inf at the pairs the mask excludes (else from 0)
    //   sm(H)    P = exp2(S c - lse2) and dS = P (dP - delta) in registers
    //            (16 elements per lane), rounded to bf16; a masked pair has
    //            S = -inf and c > 0, so its P is exactly 0
    //   dKV(H)   dV^T += dO^T P and dK^T += Q^T dS (NB MFMAs, A = transposing
    //            LDS reads of dO / Q)
    // and the kernel runs them as a pipeline: phase H issues SdP(H+1), sm(H)
    // and dKV(H-1), three independent streams, so the exponentials are spread
    // over all the MFMAs and no phase waits on a result of its own.  Phase 2u
    // reads slots u and u-1, phase 2u+1 slots u+1 and u; the workgroup
    // barrier of step u sits between them (see below).  Each MFMA's A operand
    // is read from LDS AHEAD MFMAs before it.
    constexpr int NA = 2 * C::KS;   // SdP MFMAs of a half
    constexpr int NB = 4 * C::DB;   // dKV MFMAs of a half
    static_assert(NA == NB, "phase slots");
    constexpr int AHEAD = 4;
    constexpr int RING = AHEAD + 1;

    f32x16 sa[2], pa[2];        // S and dP - delta of the last halves, by m
    bf16x8 pb[2][2], sb[2][2];  // P and dS (bf16) of the last halves, by m
    const f32x16 zero = {};
  #pragma unroll
    for (int m = 0; m < 2; ++m)
  #pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        pb[m][m2] = bf16x8{};
        sb[m][m2] = bf16x8{};
      }

    // One phase.  SN/MN: slot and m of the SdP half (tile tn); SC/MC: of the
    // softmax half; SP/MP: of the dKV half.  DO_SDP / DO_SM / DO_KV switch the
    // three streams (pipeline fill and drain).
    auto phase = [&](auto sn_c, auto mn_c, auto sc_c, auto mc_c, auto sp_c,
                     auto mp_c, auto do_sdp_c, auto do_sm_c, auto do_kv_c,
                     auto full_c, int tn) __attribute__((always_inline)) {
      constexpr bool FULLT = decltype(full_c)::value;  // tile tn known full
      constexpr int MN = decltype(mn_c)::value, MC = decltype(mc_c)::value;
      constexpr int MP = decltype(mp_c)::value;
      constexpr bool DO_SDP = decltype(do_sdp_c)::value;
      constexpr bool DO_SM = decltype(do_sm_c)::value;
      constexpr bool DO_KV = decltype(do_kv_c)::value;
      const uint16_t* Qn = qslot(sn_c);
      const uint16_t* On = oslot(sn_c);
      const float* Dn = dslot(sn_c);
      const float* Lc = lslot(sc_c);
      const uint16_t* Qp = qslot(sp_c);
      const uint16_t* Op = oslot(sp_c);

      // the MFMAs of the phase in issue order: with both streams on, even
      // slots are SdP and odd ones dKV
      constexpr int NS = (DO_SDP ? NA : 0) + (DO_KV ? NB : 0);
      constexpr bool BOTH = DO_SDP && DO_KV;
      auto fetch = [&](auto i_c) __attribute__((always_inline)) -> bf16x8 {
        constexpr int i = decltype(i_c)::value;
        constexpr int k = BOTH ? i / 2 : i;
        if constexpr (BOTH ? (i % 2 == 0) : DO_SDP) {
          constexpr int ks = k / 2;
          const uint16_t* tb = (k % 2 == 0) ? Qn : On;
          return *reinterpret_cast<const bf16x8*>(tb + aoff[MN][ks]);
        } else {
          constexpr int m2 = k / (2 * C::DB), db = (k % (2 * C::DB)) / 2;
          const uint16_t* tb = (k % 2 == 0) ? Op : Qp;
          constexpr int c0 = (32 * MP + 8 * m2) * D;
          return tr_pair(tb + toff[0][db] + c0, tb + toff[1][db] + c0 + 4 * D);
        }
      };
      // S of the SdP half starts from its mask (0 or -inf), dP from -delta of
      // its rows, so that the accumulator ends at dP - delta
      f32x16 s0 = zero, nd0;
      if constexpr (DO_SDP) {
  #pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 d4 =
              *reinterpret_cast<const f32x4*>(Dn + MN * 32 + 16 * g + 4 * q4);
  #pragma unroll
          for (int e = 0; e < 4; ++e) nd0[4 * q4 + e] = d4[e];
        }
        if (!FULLT && !tile_full(tn)) {
          // rows 32 MN + 16 g + r of tile tn, allowed in [rlo, rhi)
          const int base = tn * kRT + MN * 32 + 16 * g;
          const int mlo = rlo - base, mhi = rhi - base;
  #pragma unroll
          for (int r = 0; r < 16; ++r)
            s0[r] = (r >= mlo && r < mhi) ? 0.f : -INFINITY;
        }
      }
      auto mfma = [&](auto i_c, const bf16x8& a) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value;
        constexpr int k = BOTH ? i / 2 : i;
        if constexpr (BOTH ? (i % 2 == 0) : DO_SDP) {
          constexpr int ks = k / 2;
          if constexpr (k % 2 == 0)
            sa[MN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, kf[ks], ks == 0 ? s0 : sa[MN], 0, 0, 0);
          else
            pa[MN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, vf[ks], ks == 0 ? nd0 : pa[MN], 0, 0, 0);
        } else {
          constexpr int m2 = k / (2 * C::DB), db = (k % (2 * C::DB)) / 2;
          if constexpr (k % 2 == 0)
            dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[MP][m2],
                                                              dva[db], 0, 0, 0);
          else
            dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[MP][m2],
                                                              dka[db], 0, 0, 0);
        }
      };

      // softmax of rows 32 MC + 16 g + r of the softmax half (lane = key)
      float pvv[16], dsv[16];
      f32x4 l4;
      auto element = [&](auto r_c) __attribute__((always_inline)) {
        constexpr int r = decltype(r_c)::value;
        if constexpr (r % 4 == 0)
          l4 = *reinterpret_cast<const f32x4*>(Lc + MC * 32 + 16 * g + r);
        const float pr = __builtin_amdgcn_exp2f(fmaf(sa[MC][r], cc, -l4[r % 4]));
        pvv[r] = pr;
        dsv[r] = pr * pa[MC][r];
        if constexpr (r % 8 == 7) {
          constexpr int m2 = r / 8;
          f32x8 x, y;
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[e] = pvv[8 * m2 + e];
            y[e] = dsv[8 * m2 + e];
          }
          pb[MC][m2] = __builtin_convertvector(x, bf16x8);
          sb[MC][m2] = __builtin_convertvector(y, bf16x8);
        }
      };

      if constexpr (NS > 0) {
        bf16x8 ring[RING];
        static_for<0, (AHEAD < NS ? AHEAD : NS)>(
            [&](auto i_c) __attribute__((always_inline)) {
              ring[decltype(i_c)::value] = fetch(i_c);
            });
        static_for<0, NS>([&](auto i_c) __attribute__((always_inline)) {
          constexpr int i = decltype(i_c)::value;
          if constexpr (i + AHEAD < NS)
            ring[(i + AHEAD) % RING] = fetch(ic<i + AHEAD>());
          mfma(i_c, ring[i % RING]);
          // the softmax's 16 elements spread over the phase's MFMAs
          if constexpr (DO_SM) {
            static_for<i * 16 / NS, (i + 1) * 16 / NS>(
                [&](auto e_c) __attribute__((always_inline)) {
                  element(e_c);
                });
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
        });
      } else if constexpr (DO_SM) {
        static_for<0, 16>([&](auto e_c) __attribute__((always_inline)) {
          element(e_c);
        });
      }
    };

    using T = std::true_type;
    using F = std::false_type;
    auto tile_of_step = [&](int u) { return t_last - u / p.G; };
    // Step u (slot S = u % 3): phase 2u, then each wave waits for its loads of
    // step u + 1 and takes the barrier, then issues the loads of step u + 2
    // into slot (u + 2) % 3 (last read in phase 2u, by dKV(2u - 1)), then
    // phase 2u + 1.  Before step 0: the loads of steps 0 and 1, slot 2's tiles
    // zeroed (phase 0's dKV(-1) reads them, with zero P and dS), the barrier,
    // and SdP(0).  After the last step n - 1: dKV(2n - 1).  Phase 2n - 1 also
    // forms SdP(2n) from a stale slot; that result is never used.
    if (nsteps > 0) {
      issue(ic<0>(), 0);
      if (1 < nsteps) issue(ic<1>(), 1);
      {
        constexpr int CHUNKS = C::TILE / 8;  // 16-byte chunks per tile
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int c = tid; c < CHUNKS; c += 64 * NW) {
          *reinterpret_cast<u32x4*>(Qs2 + 8 * c) = z;
          *reinterpret_cast<u32x4*>(Os2 + 8 * c) = z;
        }
      }
      wait_vm0();
      __syncthreads();
      phase(ic<0>(), ic<0>(), ic<0>(), ic<0>(), ic<0>(), ic<0>(), T(), F(), F(),
            F(), tile_of_step(0));
      // step u; `full` (compile time): tiles u and u + 1 are wholly allowed
      // for every key of the wave and u + 2 < nsteps, so that neither phase
      // builds a mask and the loads need no test
      auto step = [&](auto s_c, auto full_c, int u)
                      __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        constexpr int S1 = (S + 1) % 3, S2 = (S + 2) % 3;
        constexpr bool FULLS = decltype(full_c)::value;
        phase(ic<S>(), ic<1>(), ic<S>(), ic<0>(), ic<S2>(), ic<1>(), T(), T(),
              T(), full_c, tile_of_step(u));
        wait_vm0();
        barrier_nofence();
        if (FULLS || u + 2 < nsteps) issue(ic<S2>(), u + 2);
        phase(ic<S1>(), ic<0>(), ic<S>(), ic<1>(), ic<S>(), ic<0>(), T(), T(),
              T(), full_c, tile_of_step(u + 1));
      };
      // The full tiles [f0, f1) are the steps [ua, ub) (tiles go down as u
      // goes up); lean steps [la, lb), run in triples from a multiple of 3
      // (the ring slot of step u is u % 3) in a loop of their own
      const int f0 = (w_lo_max + kRT - 1) / kRT, f1 = w_hi_min / kRT;
      const int ua = p.G * max(0, t_last - f1 + 1);
      const int ub = p.G * max(0, t_last - f0 + 1);
      const int la = ua, lb = min(ub - 1, nsteps - 2);
      const int lp0 = (la + 2) / 3 * 3;
      const int lp1 = lb - lp0 >= 3 ? lp0 + (lb - lp0) / 3 * 3 : lp0;
      int u = 0;
      for (; u + 3 <= (lp1 > lp0 ? lp0 : nsteps); u += 3) {
        step(ic<0>(), F(), u);
        step(ic<1>(), F(), u + 1);
        step(ic<2>(), F(), u + 2);
      }
      if (lp1 > lp0) {
        for (; u < lp1; u += 3) {
          step(ic<0>(), T(), u);
          step(ic<1>(), T(), u + 1);
          step(ic<2>(), T(), u + 2);
        }
        for (; u + 3 <= nsteps; u += 3) {
          step(ic<0>(), F(), u);
          step(ic<1>(), F(), u + 1);
          step(ic<2>(), F(), u + 2);
        }
      }
      if (u < nsteps) step(ic<0>(), F(), u++);
      if (u < nsteps) step(ic<1>(), F(), u++);
      // dKV(2n - 1): slot (n - 1) % 3
      const int sl = (nsteps - 1) % 3;
      if (sl == 0)
        phase(ic<0>(), ic<0>(), ic<0>(), ic<0>(), ic<0>(), ic<1>(), F(), F(), T(),
              F(), 0);
      else if (sl == 1)
        phase(ic<1>(), ic<0>(), ic<1>(), ic<0>(), ic<1>(), ic<1>(), F(), F(), T(),
              F(), 0);
      else
        phase(ic<2>(), ic<0>(), ic<2>(), ic<0>(), ic<2>(), ic<1>(), F(), F(), T(),
              F(), 0);
    }
  }

  // dK = scale * dK^T accumulated, dV; keys past the valid length get 0
  if (j < p.Nk) {
    const bool kv_ok = j < s.L;
    uint16_t* dkr = p.dk + kv_base + (size_t)j * D;
    uint16_t* dvr = p.dv + kv_base + (size_t)j * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int quad = 0; quad < 4; ++quad) {
        f32x4 x, y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = kv_ok ? dka[db][4 * quad + e] * p.scale : 0.f;
          y[e] = kv_ok ? dva[db][4 * quad + e] : 0.f;
        }
        const int col = db * 32 + quad * 8 + 4 * g;
        *reinterpret_cast<bf16x4*>(dkr + col) =
            __builtin_convertvector(x, bf16x4);
        *reinterpret_cast<bf16x4*>(dvr + col) =
            __builtin_convertvector(y, bf16x4);
      }
  }
}

// ---------------------------------------------------------------------------
// bwd_dq

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(
    BwdParams p) {
  using C = BCfg<D>;
  constexpr int QB = kWR * NW;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[C::TILE];
  auto kslot = [&](auto s) -> uint16_t* {
    if constexpr (decltype(s)::value == 0) return Ks0; else return Ks1;
  };
  auto vslot = [&](auto s) -> uint16_t* {
    if constexpr (decltype(s)::value == 0) return Vs0; else return Vs1;
  };

  // (batch, K/V head, query block, head of the group): the order of
  // block_order.h, as for the forward (whole groups per XCD, causal blocks
  // heaviest first across an XCD's groups)
  const BlockPos bpos = block_pos(blockIdx.x, p.order);
  const int qb = bpos.qb;
  const int b = bpos.b;
  const int hk = bpos.hk;
  const int hh = bpos.hh;
  const int h = hk * p.G + hh;
  const Seq s = seq_of(p.seqlens, p.Nq, p.Nk, b);
  auto row_keys = [&](bool live, int pos) {
    return keys_of_row(s, p.causal, p.window, p.window_right, p.sinks, live,
                       pos);
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int q0 = qb * QB;
  const int qw0 = q0 + wave * kWR;
  const int qi = qw0 + ql;
  const bool qlive = qi < s.Lq;
  const RowKeys rk = row_keys(qlive, qi + s.off);

  // the workgroup's tiles: sink tiles [0, ts1), then window tiles
  // [tw0, tw1), merged into one run when they meet; step u visits tile_of(u)
  const int rows_end = min(q0 + QB, s.Lq);
  int nA = 0, tB0 = 0, nt = 0;
  if (rows_end > q0) {
    const RowKeys first = row_keys(true, q0 + s.off);
    const RowKeys last = row_keys(true, rows_end - 1 + s.off);
    int tw0 = first.lo / kRT, tw1 = (last.hw + kRT - 1) / kRT;
    if (last.hw <= first.lo) tw0 = tw1 = 0;
    const int ts1 = (last.sk + kRT - 1) / kRT;
    if (ts1 >= tw0) {
      nA = max(ts1, tw1);
      nt = nA;
    } else {
      nA = ts1;
      tB0 = tw0;
      nt = ts1 + (tw1 - tw0);
    }
  }
  auto tile_of = [&](int u) { return u < nA ? u : tB0 + (u - nA); };

  // over the wave's live rows: hull and intersection of their key sets
  const int wend = min(qw0 + kWR, s.Lq);
  const bool wlive = wend > qw0;
  RowKeys wf = {0, 0, 0, 0}, wl = {0, 0, 0, 0};
  if (wlive) {
    wf = row_keys(true, qw0 + s.off);
    wl = row_keys(true, wend - 1 + s.off);
  }
  auto wave_needs = [&](int t) {
    const int j0 = t * kRT;
    return wlive && ((j0 < wl.hw && j0 + kRT > wf.lo) || j0 < wl.sk);
  };
  auto tile_full = [&](int t) {
    const int j0 = t * kRT;
    return (j0 >= wl.lo && j0 + kRT <= wf.hw) || j0 + kRT <= wf.sk;
  };

  // Q and dO of this lane's row as B operands; lse and delta of the row
  const size_t bh = (size_t)b * p.Hq + h;
  // S c is formed with c > 0 (the mask relies on -inf c = -inf): for a
  // negative scale Q is negated on load (its only use is S) and c flipped;
  // scale 0 takes a tiny positive c, under which every allowed pair weighs
  // the same
  const bool qneg = p.c < 0.f;
  const float cc = qneg ? -p.c : (p.c > 0.f ? p.c : 1e-30f);
  const unsigned qsign = qneg ? 0x80008000u : 0u;
  bf16x8 qf[C::KS], of[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (qlive) {
      a = *reinterpret_cast<const u32x4*>(p.q + (bh * p.Nq + qi) * D +
                                          16 * ks + 8 * g);
      c = *reinterpret_cast<const u32x4*>(p.dout + (bh * p.Nq + qi) * D +
                                          16 * ks + 8 * g);
    }
    a ^= qsign;
    qf[ks] = __builtin_bit_cast(bf16x8, a);
    of[ks] = __builtin_bit_cast(bf16x8, c);
  }
  const float l2 = qlive ? p.lse2[bh * p.Nqp + qi] : INFINITY;
  const float ndl = qlive ? p.delta[bh * p.Nqp + qi] : 0.f;

  f32x16 dqa[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[db][r] = 0.f;

  int aoff[2][C::KS];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) aoff[mb][ks] = a_off<D>(lane, mb, ks);
  int toff[2][C::DB];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      toff[half][db] = tr_off<D>(lane, half, db);

  const size_t kv_base = (size_t)(b * p.Hkv + hk) * p.Nk * D;
  // this wave's tile loads: wave w issues loads w, w + NW, ... of the K tile
  // and the same of the V tile (LOADS is a multiple of NW), at the same
  // per-lane offsets
  static_assert(C::LOADS % NW == 0, "loads per wave");
  constexpr int TW = C::LOADS / NW;
  unsigned toffs[TW];
#pragma unroll
  for (int m = 0; m < TW; ++m) toffs[m] = tile_src_off<D>(wave + NW * m, lane);
  const auto krs = rows_rsrc(p.k + kv_base, s.L * D * 2);
  const auto vrs = rows_rsrc(p.v + kv_base, s.L * D * 2);
  auto issue = [&](auto slot_c, int tile) {
    const int tb = tile * kRT * D * 2;
#pragma unroll
    for (int m = 0; m < TW; ++m)
      miattn_buffer_load_lds(
          krs, (lds_void*)(kslot(slot_c) + (wave + NW * m) * 512), 16,
          toffs[m] + tb, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < TW; ++m)
      miattn_buffer_load_lds(
          vrs, (lds_void*)(vslot(slot_c) + (wave + NW * m) * 512), 16,
          toffs[m] + tb, 0, 0, 0);
  };

  // compute(full, slot, t): tile t's products; `full` (compile time) when
  // every row of the wave sees the whole tile
  auto compute = [&](auto full_c, auto slot_c, int t) {
    constexpr bool FULL = decltype(full_c)::value != 0;
    if (!FULL && !wave_needs(t)) return;
    const uint16_t* Kt = kslot(slot_c);
    const uint16_t* Vt = vslot(slot_c);
    // S^T = K Q^T and dP^T = V dO^T: lane (query, g) holds keys
    // mb*32 + 16g + r of the tile.  On a tile that needs the mask, S^T
    // starts from -inf at the pairs the mask excludes (else from 0): with
    // c > 0 their P is then exactly 0.
    const int j0 = t * kRT;
    f32x16 sa[2], pa[2];
    const f32x16 zero = {};
    if constexpr (!FULL) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) sa[mb] = zero;
    }
    if (!FULL && !tile_full(t)) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = j0 + mb * 32 + 16 * g + r;
          const bool ok =
              (jj < rk.hc) & (((jj >= rk.lo) & (jj < rk.hw)) | (jj < rk.sk));
          sa[mb][r] = ok ? 0.f : -INFINITY;
        }
    }
    // the 4 KS MFMAs (ks, mb, S^T or dP^T), each A operand read from LDS
    // two MFMAs ahead
    constexpr int NS = 4 * C::KS;
    auto fetch = [&](auto i_c) __attribute__((always_inline)) -> bf16x8 {
      constexpr int i = decltype(i_c)::value;
      constexpr int ks = i / 4, mb = (i / 2) % 2;
      return *reinterpret_cast<const bf16x8*>((i % 2 == 0 ? Kt : Vt) +
                                              aoff[mb][ks]);
    };
    bf16x8 ring[3];
    ring[0] = fetch(ic<0>());
    ring[1] = fetch(ic<1>());
    static_for<0, NS>([&](auto i_c) __attribute__((always_inline)) {
      constexpr int i = decltype(i_c)::value;
      constexpr int ks = i / 4, mb = (i / 2) % 2;
      if constexpr (i + 2 < NS) ring[(i + 2) % 3] = fetch(ic<i + 2>());
      if constexpr (i % 2 == 0)
        sa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            ring[i % 3], qf[ks], (FULL && ks == 0) ? zero : sa[mb], 0, 0, 0);
      else
        pa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            ring[i % 3], of[ks], ks == 0 ? zero : pa[mb], 0, 0, 0);
    });
    // dS^T = P (dP - delta) of keys 32 mb + 16 g + r, in bf16
    bf16x8 sb[2][2];
    float dsv[16];
    auto element = [&](auto mb_c, auto r_c) __attribute__((always_inline)) {
      constexpr int mb = decltype(mb_c)::value, r = decltype(r_c)::value;
      const float pr = __builtin_amdgcn_exp2f(fmaf(sa[mb][r], cc, -l2));
      dsv[r] = pr * (pa[mb][r] + ndl);
      if constexpr (r % 8 == 7) {
        constexpr int m2 = r / 8;
        f32x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = dsv[8 * m2 + e];
        sb[mb][m2] = __builtin_convertvector(y, bf16x8);
      }
    };
    static_for<0, 16>([&](auto r_c) __attribute__((always_inline)) {
      element(ic<0>(), r_c);
    });
    // dQ^T += K^T dS^T over the tile's 64 keys (4 DB MFMAs, (mb, m2, db)),
    // A operands read two MFMAs ahead; the dS^T of keys 32 .. 63 is formed
    // between the MFMAs over keys 0 .. 31
    constexpr int NQ = 4 * C::DB;
    auto fetch_q = [&](auto i_c) __attribute__((always_inline)) -> bf16x8 {
      constexpr int i = decltype(i_c)::value;
      constexpr int mb = i / (2 * C::DB), m2 = (i / C::DB) % 2,
                    db = i % C::DB;
      constexpr int c0 = (32 * mb + 8 * m2) * D;
      return tr_pair(Kt + toff[0][db] + c0, Kt + toff[1][db] + c0 + 4 * D);
    };
    bf16x8 qring[3];
    qring[0] = fetch_q(ic<0>());
    qring[1] = fetch_q(ic<1>());
    static_for<0, NQ>([&](auto i_c) __attribute__((always_inline)) {
      constexpr int i = decltype(i_c)::value;
      constexpr int mb = i / (2 * C::DB), m2 = (i / C::DB) % 2,
                    db = i % C::DB;
      if constexpr (i + 2 < NQ) qring[(i + 2) % 3] = fetch_q(ic<i + 2>());
      dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qring[i % 3],
                                                        sb[mb][m2], dqa[db], 0,
                                                        0, 0);
      if constexpr (i < NQ / 2) {
        static_for<i * 32 / NQ, (i + 1) * 32 / NQ>(
            [&](auto r_c) __attribute__((always_inline)) {
              element(ic<1>(), r_c);
            });
      }
    });
  };

  if (nt > 0) {
    issue(ic<0>(), tile_of(0));
    wait_vm0();
    barrier_nofence();
    auto step = [&](auto slot_c, int u) {
      constexpr int S = decltype(slot_c)::value;
      if (u + 1 < nt) issue(ic<1 - S>(), tile_of(u + 1));
      compute(ic<0>(), slot_c, tile_of(u));
      wait_vm0();
      barrier_nofence();
    };
    // Interior steps [la, lb) of the longer run: every row of the wave sees
    // the whole tile, and the next tile belongs to the run.  Such a step is
    // the one above with every decision known (tile u + loff, no test, no
    // mask, S started from the zero operand).
    int la = 0, lb = 0;
    const int s0 = nt > nA ? nA : 0, s1 = nt > nA ? nt : nA;
    const int loff = nt > nA ? tB0 - nA : 0;
    if (wlive) {
      const int f0 = (wl.lo + kRT - 1) / kRT;  // first tile left-full
      const int f1 = wf.hw / kRT;              // tiles below: right-full
      la = max(s0, f0 - loff);
      lb = min(s1 - 1, f1 - loff);
    }
    auto lean = [&](auto slot_c, int u) {
      constexpr int S = decltype(slot_c)::value;
      issue(ic<1 - S>(), u + 1 + loff);
      compute(ic<1>(), slot_c, u + loff);
      wait_vm0();
      barrier_nofence();
    };
    // lean pairs in a loop of their own, between the general steps
    const int lp0 = la + (la & 1);
    const int lp1 = lp0 + 1 < lb ? lp0 + ((lb - lp0) & ~1) : lp0;
    int u = 0;
    for (; u < (lp1 > lp0 ? lp0 : nt); u += 2) {
      step(ic<0>(), u);
      if (u + 1 < nt) step(ic<1>(), u + 1);
    }
    if (lp1 > lp0) {
      for (; u < lp1; u += 2) {
        lean(ic<0>(), u);
        lean(ic<1>(), u + 1);
      }
      for (; u < nt; u += 2) {
        step(ic<0>(), u);
        if (u + 1 < nt) step(ic<1>(), u + 1);
      }
    }
  }

  // dQ = scale * dQ^T accumulated; dead rows get 0
  if (qi < p.Nq) {
    uint16_t* dqr = p.dq + (bh * p.Nq + qi) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int quad = 0; quad < 4; ++quad) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = qlive ? dqa[db][4 * quad + e] * p.scale : 0.f;
        *reinterpret_cast<bf16x4*>(dqr + db * 32 + quad * 8 + 4 * g) =
            __builtin_convertvector(x, bf16x4);
      }
  }
}

constexpr int kDkdvNW = 4;   // 128 keys per workgroup
static_assert(kDkdvNW == lanes::kBwdWaves, "shared lane layout");
// dQ: 128 rows per workgroup and two workgroups per CU (two waves per SIMD
// from independent workgroups, which drift out of phase; one 8-wave
// workgroup per CU was 5-10% slower at d=128)
constexpr int kDqNW128 = 4;
constexpr int kDqNW64 = 4;
static_assert(kDqNW128 == lanes::kBwdWaves && kDqNW64 == lanes::kBwdWaves,
              "shared lane layout");

template <int D, int NWK, int NWQ>
hipError_t launch_all(BwdParams p, hipStream_t st) {
  const long long rows = (long long)p.B * p.Hq * p.Nqp;
  const long long waves = (rows * D / 8 + 63) / 64;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((waves + 3) / 4)),
                     dim3(256), 0, st, p);
  BwdParams a = p;
  a.nblk = (p.Nk + kWR * NWK - 1) / (kWR * NWK);
  a.total = p.B * p.Hkv * a.nblk;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, NWK, D == 128>), dim3(a.total),
                     dim3(64 * NWK), 0, st, a);
  BwdParams c = p;
  c.nblk = (p.Nq + kWR * NWQ - 1) / (kWR * NWQ);
  c.total = p.B * p.Hq * c.nblk;
  c.order = make_block_order(p.B, p.Hkv, p.G, c.nblk, p.causal != 0,
                             2LL * p.Nk * D * 2, 32 * 2);
  hipLaunchKernelGGL((bwd_dq_kernel<D, NWQ>), dim3(c.total), dim3(64 * NWQ),
                     0, st, c);
  return hipGetLastError();
}

}  // namespace bwd_impl

using namespace bwd_impl;

size_t bwd_workspace_bytes(const Problem& pr) {
  const size_t nqp = (size_t)((pr.Nq + kRT - 1) / kRT) * kRT;
  return 2 * (size_t)pr.B * pr.Hq * nqp * sizeof(float);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse,
                           void* dq, void* dk, void* dv, const Problem& pr,
                           void* ws, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.seqlens = pr.seqlens;
  p.B = pr.B;
  p.Hq = pr.Hq;
  p.Hkv = pr.Hkv;
  p.Nq = pr.Nq;
  p.Nk = pr.Nk;
  p.Nqp = (pr.Nq + kRT - 1) / kRT * kRT;
  p.G = pr.Hq / pr.Hkv;
  p.causal = pr.causal;
  p.window = pr.window;
  p.window_right = pr.window_right;
  p.sinks = pr.sinks;
  p.scale = pr.scale;
  p.c = pr.scale * 1.4426950408889634f;
  const size_t n = (size_t)pr.B * pr.Hq * p.Nqp;
  p.lse2 = static_cast<float*>(ws);
  p.delta = p.lse2 + n;
  p.nblk = 0;
  p.total = 0;
  if (pr.d == 128) return launch_all<128, kDkdvNW, kDqNW128>(p, stream);
  return launch_all<64, kDkdvNW, kDqNW64>(p, stream);
}

}  // namespace miattn
