// FP8 attention on gfx950: block quantization with incoherent processing,
// and a forward kernel whose two matrix products run on FP8 matrix cores.
//
// What is computed (the FlashAttention-3 review page's FP8 sections: block
// quantization and incoherent processing):
//   Q'' = Q D H, K'' = K D H      (optional; D = diag(signs), H the
//                                  Sylvester Hadamard matrix, entries +-1:
//                                  Q'' K''^T = d Q K^T, the softmax scale is
//                                  divided by d)
//   every 64-row block of Q'', K'', V of one (batch, head) is scaled by
//   448 / amax (amax over its valid rows) and rounded to E4M3; the block's
//   scale amax / 448 is kept
//   O = softmax(scale * deq(Q) deq(K)^T + mask) deq(V), lse as for attn_fwd
// E4M3 is the OCP variant the hardware converts to: round to nearest even,
// 448 the largest finite value.
//
// Storage of the quantized operands (bytes; Nkp = Nk rounded up to 64):
//   q8  [B][Hq][Nq][d]          sq [B][Hq][ceil(Nq/64)]
//   k8  [B][Hkv][Nkp][d]        sk [B][Hkv][Nkp/64]
//   v8t [B][Hkv][Nkp/64][d][64] sv [B][Hkv][Nkp/64]   (each 64-key tile of V
//                                                      stored transposed)
// Rows past the valid length (and dead query rows) hold code 0.
//
// Quantizer: one workgroup per 64-row block.  A row of d values is spread
// over a wavefront, d/64 per lane; the Hadamard transform runs as butterfly
// stages of width 1, 2, ..., d/2 (within a lane while the width is below
// d/64, else with the lane whose index differs in one bit), in float32, in
// that order, so every value is the same float32 the reference computes.
// Block amax by wave then workgroup reduction; codes by v_cvt_pk_fp8_f32.
//
// Forward kernel: the bf16 forward kernel's decomposition (wave = 32 query
// rows, 64-key tiles, transposed products) with FP8 operands:
//   S^T = K Q''^T      v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales),
//                      A = K rows from LDS, B = Q'' rows held in registers
//   p = exp2(S^T * sq * sk_t * c - m) with the running maximum m moved once
//   a score passes it by 2^0.5; w = p * (sv_t / sv_max) * 256 is rounded to
//   E4M3 (the tile's V scale folded into P; 256 keeps small weights out of
//   the subnormal range, and p <= 2^0.5 keeps w below 448)
//   O^T += V^T W^T     A = V^T rows of the transposed tile, B = W^T straight
//                      from the S^T accumulator layout
//   O = O^T * sv_max / 256 / l
// Tiles come by direct-to-LDS buffer loads into two ring slots; the 16-byte
// chunks of every LDS row are permuted by an XOR of row bits so that the
// operand reads are free of bank conflicts.  Workgroups of 4 wavefronts (128
// query rows), two per CU: their barriers are independent, so the two waves
// on each SIMD drift out of phase and one's softmax overlaps the other's
// matrix products (one 8-wavefront workgroup per CU ran 12% slower).  Blocks
// are dealt to the XCDs in the bf16 kernel's order (block_order.h), and the
// steps in which a wave needs all of two consecutive tiles run in a loop of
// their own, with no per-step test.
#include "kernels.h"

#include <cmath>
#include <type_traits>

#include "block_order.h"
#include "tail_queue.h"
#include "device_common.h"

namespace miattn {
namespace fp8_impl {

using namespace dev;

// max(x, x of the lane 32 apart) on the VALU: v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second,
// both copies of x; two distinct registers, since the builtin given one
// value twice was folded to a single result.
__device__ inline float half_swap_max(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBlk = 64;        // rows of a quantization block and of a tile
constexpr int kWR = 32;         // query rows per wavefront
// Lazy-rescale threshold (log2 units): a probability may reach 2^kTau
// before the running maximum moves, and 2^kTau * kPScale must stay within
// E4M3's 448.
constexpr float kTau = 0.5f;
constexpr float kE4M3Max = 448.0f;
constexpr float kPScale = 256.0f;

// Chunk permutations (16-byte chunks): K tile rows are 128 bytes (d = 128)
// or 64 bytes (d = 64) and are read 16 rows at a time in mfma_row order;
// V^T tile rows are 64 bytes read 16 consecutive rows at a time.
template <int D>
__device__ inline int swz_k(int r) {
  return lanes::fp8_swz_k(D, r);
}
__device__ inline int swz_v(int r) { return lanes::fp8_swz_v(r); }

// ---------------------------------------------------------------------------
// quantizer

struct QuantParams {
  const uint16_t* x;   // bf16 [B][H][N][d]
  uint8_t* codes;      // layout below
  float* scales;       // [B][H][nblk]
  const int* seqlens;
  const signed char* signs;  // d entries (+-1) or null: no rotation
  int B, H, N, d, Nq, Nk;    // Nq, Nk: the attention problem's sizes
  int is_q;            // rows valid: live query rows (else the valid length)
  int transposed;      // codes as [B][H][nblk][d][64] (V), else [B][H][Npad][d]
  int Npad;            // rows per head in `codes` (N, or Nk rounded to 64)
  int nblk;            // blocks per head
  int mode;            // 0: block scale; 1: amax only; 2: preset amax
};

// Up to three tensors quantized by one launch: blocks [first[i], first[i+1])
// (first[3] = the grid) belong to tensor i.
struct QuantSet {
  QuantParams t[3];
  int first[4];
};

// x of the lane whose index differs from this one's in bit LB (LB = 1, 2,
// 4, 8): DPP quad permutations for 1 and 2, a rotation by 8 within the
// 16-lane row for 8 (the same pairing), a swizzle for 4.
template <int LB>
__device__ inline float lane_xor(float x) {
  const int i = __float_as_int(x);
  int r;
  if constexpr (LB == 1)
    r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true);  // [1,0,3,2]
  else if constexpr (LB == 2)
    r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
  else if constexpr (LB == 8)
    r = __builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, true);  // row_ror:8
  else
    r = __builtin_amdgcn_ds_swizzle(i, 0x1F | (LB << 10));  // xor LB
  return __int_as_float(r);
}

// mode 0: codes and scale from the block's own amax; mode 1: writes the
// block's amax to scales[] and nothing else; mode 2: reads amax from
// scales[] (all blocks of the tensor set to one value), writes codes and the
// scale amax / 448.
// Layout of the work: a workgroup of 4 waves takes one block of 64 rows,
// 16 rows a wave.  A row is D / 8 lanes of 8 values (16-byte loads, so one
// wave instruction reads RPI whole rows); the butterflies of width 1, 2 and 4
// stay inside a lane, those of width 8 .. D/2 pair lanes of the same row.
// The levels run in the same order (width 1 first) as one lane holding a
// whole row would run them, so every value goes through the same float32
// operations.
template <int D>
__global__ __launch_bounds__(256) void fp8_quant_kernel(QuantSet set) {
  constexpr int LPR = D / 8;     // lanes per row
  constexpr int RPI = 64 / LPR;  // rows per wave instruction
  constexpr int NI = 16 / RPI;   // instructions for a wave's 16 rows
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * kBlk];
  const int bid = blockIdx.x;
  const int ti = bid >= set.first[2] ? 2 : (bid >= set.first[1] ? 1 : 0);
  const QuantParams& p = set.t[ti];
  const int lbid = bid - set.first[ti];
  const int blk = lbid % p.nblk;
  const int bh = lbid / p.nblk;
  const int b = bh / p.H;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane / LPR;  // row of the instruction's group
  const int cl = lane % LPR;   // 8-value chunk of the row
  const Seq s = seq_of(p.seqlens, p.Nq, p.Nk, b);
  const int valid = p.is_q ? s.Lq : s.L;
  const int r0 = blk * kBlk;

  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    sg[e] = p.signs ? (float)p.signs[cl * 8 + e] : 1.0f;

  // rows r0 + wave*16 + i*RPI + sub: load, rotate, track |max|
  float v[NI][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = r0 + wave * 16 + i * RPI + sub;
    const bool ok = r < valid && r < p.N;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (ok)
      raw = *reinterpret_cast<const u32x4*>(p.x + ((size_t)bh * p.N + r) * D +
                                            cl * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      v[i][2 * w] = __uint_as_float(raw[w] << 16);
      v[i][2 * w + 1] = __uint_as_float(raw[w] & 0xffff0000u);
    }
    if (p.signs) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] *= sg[e];
      // butterflies of width h: element j pairs with j ^ h; the lower one
      // becomes a + b, the upper one a - b
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & h) == 0) {
            const float a = v[i][e], c = v[i][e + h];
            v[i][e] = a + c;
            v[i][e + h] = a - c;
          }
      // widths 8 .. D/2: the partner lane (same row) differs in bit h / 8
      static_for<0, 5>([&](auto k_c) {
        constexpr int LB = 1 << decltype(k_c)::value;
        if constexpr (8 * LB < D) {
          const bool upper = (cl & LB) != 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float o = lane_xor<LB>(v[i][e]);
            v[i][e] = upper ? o - v[i][e] : v[i][e] + o;
          }
        }
      });
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
  }
  amax = wave_maxf(amax);
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float* sp = p.scales + (size_t)bh * p.nblk + blk;
  if (p.mode == 1) {
    if (threadIdx.x == 0) *sp = amax;
    return;
  }
  if (p.mode == 2) {
    amax = *sp;  // every thread reads the preset amax before it is replaced
    __syncthreads();
  }
  const float mul = amax > 0.f ? kE4M3Max / amax : 0.f;
  if (threadIdx.x == 0) *sp = amax / kE4M3Max;

  // codes: 8 bytes a lane and row, row-major, or through LDS into the
  // transposed tile
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int rl = wave * 16 + i * RPI + sub;
    const int r = r0 + rl;
    unsigned w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      w[h] = __builtin_amdgcn_cvt_pk_fp8_f32(v[i][4 * h] * mul,
                                             v[i][4 * h + 1] * mul, 0u, false);
      w[h] = __builtin_amdgcn_cvt_pk_fp8_f32(v[i][4 * h + 2] * mul,
                                             v[i][4 * h + 3] * mul, w[h], true);
    }
    if (p.transposed) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tile[(cl * 8 + e) * kBlk + rl] = (uint8_t)(w[e / 4] >> (8 * (e % 4)));
    } else if (r < p.Npad) {
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      uint8_t* dst = p.codes + ((size_t)bh * p.Npad + r) * D + cl * 8;
      *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
    }
  }
  if (p.transposed) {
    __syncthreads();
    uint8_t* dst = p.codes + ((size_t)bh * p.nblk + blk) * D * kBlk;
    for (int o = threadIdx.x * 16; o < D * kBlk; o += 256 * 16)
      *reinterpret_cast<u32x4*>(dst + o) =
          *reinterpret_cast<const u32x4*>(tile + o);
  }
}

// Per-tensor amax: reduces the block amaxes of one tensor and writes the
// maximum back into every block's slot (then mode 2 quantizes with it).
__global__ __launch_bounds__(256) void fp8_tensor_amax_kernel(float* scales,
                                                              int n) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, scales[i]);
  m = wave_maxf(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 256) scales[i] = m;
}

// ---------------------------------------------------------------------------
// forward

struct Fp8Params {
  const uint8_t* q8;
  const float* sq;
  const uint8_t* k8;
  const float* sk;
  const uint8_t* v8t;
  const float* sv;
  uint16_t* o;
  float* lse;
  const int* seqlens;
  int B, Hq, Hkv, Nq, Nk, Nkp, G, nqb, total;
  int causal, window, window_right, sinks;
  float c;  // |scale| * log2(e) (divided by d for rotated operands)
  unsigned qsign;  // 0x80808080 when the scale is negative: Q codes negated
  BlockOrder order;  // block -> (batch, head, query block): block_order.h
  TailQueue tail;    // lightest blocks handed out at run time: tail_queue.h
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_fp8_kernel(Fp8Params p) {
  constexpr int QB = kWR * NW;
  constexpr int KT = kBlk * D;  // bytes of a K tile and of a V^T tile
  constexpr int KS = D / 64;    // k-steps of the S product
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int LOADS = 2 * KT / 1024;  // wave loads per step (K and V^T)
  constexpr int LW = (LOADS + NW - 1) / NW;
  __shared__ __attribute__((aligned(16))) uint8_t Ks0[KT];
  __shared__ __attribute__((aligned(16))) uint8_t Ks1[KT];
  __shared__ __attribute__((aligned(16))) uint8_t Vs0[KT];
  __shared__ __attribute__((aligned(16))) uint8_t Vs1[KT];
  __shared__ float red_sv[NW];
  auto kslot = [&](auto s) -> uint8_t* {
    if constexpr (decltype(s)::value == 0) return Ks0; else return Ks1;
  };
  auto vslot = [&](auto s) -> uint8_t* {
    if constexpr (decltype(s)::value == 0) return Vs0; else return Vs1;
  };

  // block -> (batch, K/V head, query block, head of the group): the order
  // of block_order.h (whole groups per XCD, causal blocks heaviest first);
  // from p.tail.first on, the workgroups take the lightest blocks from the
  // run-time queue of tail_queue.h
  int bid = blockIdx.x;
  unsigned tail_done = 0;
  if (bid >= p.tail.first) {
    __shared__ int s_bid;
    if (threadIdx.x == 0) s_bid = tail_take(p.tail, p.order.total, &tail_done);
    __syncthreads();
    bid = s_bid;
    if (bid < 0) {
      if (threadIdx.x == 0) tail_clear(p.tail, tail_done);
      return;
    }
  }
  const BlockPos bpos = block_pos(bid, p.order);
  const int qb = bpos.qb;
  const int b = bpos.b;
  const int hk = bpos.hk;
  const int hh = bpos.hh;
  const int h = hk * p.G + hh;
  const Seq s = seq_of(p.seqlens, p.Nq, p.Nk, b);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int q0 = qb * QB;
  const int qw0 = q0 + wave * kWR;
  const int qi = qw0 + ql;
  const bool qlive = qi < s.Lq;
  const RowKeys rk = keys_of_row(s, p.causal, p.window, p.window_right,
                                 p.sinks, qlive, qi + s.off);

  // tiles of the workgroup: sink tiles, then window tiles (one run when
  // they meet); step u visits tile_of(u)
  const int rows_end = min(q0 + QB, s.Lq);
  int nA = 0, tB0 = 0, nt = 0;
  if (rows_end > q0) {
    const RowKeys f = keys_of_row(s, p.causal, p.window, p.window_right,
                                  p.sinks, true, q0 + s.off);
    const RowKeys l = keys_of_row(s, p.causal, p.window, p.window_right,
                                  p.sinks, true, rows_end - 1 + s.off);
    int tw0 = f.lo / kBlk, tw1 = (l.hw + kBlk - 1) / kBlk;
    if (l.hw <= f.lo) tw0 = tw1 = 0;
    const int ts1 = (l.sk + kBlk - 1) / kBlk;
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
  const int wend = min(qw0 + kWR, s.Lq);
  const bool wlive = wend > qw0;
  RowKeys wf = {0, 0, 0, 0}, wl = {0, 0, 0, 0};
  if (wlive) {
    wf = keys_of_row(s, p.causal, p.window, p.window_right, p.sinks, true,
                     qw0 + s.off);
    wl = keys_of_row(s, p.causal, p.window, p.window_right, p.sinks, true,
                     wend - 1 + s.off);
  }
  auto wave_needs = [&](int t) {
    const int j0 = t * kBlk;
    return wlive && ((j0 < wl.hw && j0 + kBlk > wf.lo) || j0 < wl.sk);
  };
  auto tile_full = [&](int t) {
    const int j0 = t * kBlk;
    return (j0 >= wl.lo && j0 + kBlk <= wf.hw) || j0 + kBlk <= wf.sk;
  };

  // the largest V tile scale of this (batch, K/V head): every tile's V
  // scale enters P relative to it
  const int ntk = p.Nkp / kBlk;
  const float* svh = p.sv + (size_t)(b * p.Hkv + hk) * ntk;
  const float* skh = p.sk + (size_t)(b * p.Hkv + hk) * ntk;
  float svm = 0.f;
  for (int t = tid; t < ntk; t += 64 * NW) svm = fmaxf(svm, svh[t]);
  svm = wave_maxf(svm);
  if (lane == 0) red_sv[wave] = svm;
  __syncthreads();
  svm = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) svm = fmaxf(svm, red_sv[w]);
  const float inv_svm = svm > 0.f ? kPScale / svm : 0.f;

  // Q'' of this lane's row as B operand: 32 bytes per k-step
  const size_t bhq = (size_t)b * p.Hq + h;
  i32x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 lo4 = {0u, 0u, 0u, 0u}, hi4 = {0u, 0u, 0u, 0u};
    if (qlive) {
      const uint8_t* src = p.q8 + (bhq * p.Nq + qi) * D + 64 * ks + 32 * g;
      lo4 = *reinterpret_cast<const u32x4*>(src) ^ p.qsign;
      hi4 = *reinterpret_cast<const u32x4*>(src + 16) ^ p.qsign;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[ks][e] = (int)lo4[e];
      qf[ks][4 + e] = (int)hi4[e];
    }
  }
  const float sqr = qlive ? p.sq[bhq * ((p.Nq + kBlk - 1) / kBlk) + qi / kBlk]
                          : 0.f;
  // row factor of the scores (log2 units); a zero block scale means zero
  // scores, and a tiny positive factor keeps masked scores at -inf
  const float crow = fmaxf(sqr * p.c, 1e-30f);

  // LDS operand offsets: K rows (two 16-byte chunks per k-step), V^T rows
  // (chunks g and 2 + g: keys 16g .. 16g+15 and 32+16g .. 32+16g+15)
  int koff[2][KS][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int row = mfma_row(mb * 32 + ql);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        koff[mb][ks][hf] =
            row * D + 16 * ((4 * ks + 2 * g + hf) ^ swz_k<D>(row));
  }
  int voff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int row = db * 32 + ql;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      voff[db][hf] = row * 64 + 16 * ((2 * hf + g) ^ swz_v(row));
  }

  // direct-to-LDS loads: wave load u2 = wave + NW*m; the first KT/1024 fill
  // the K tile, the rest the V^T tile; each lane's source offset in a tile
  // is fixed
  unsigned toffs[LW];
#pragma unroll
  for (int m = 0; m < LW; ++m) {
    const int u2 = wave + NW * m;
    static_assert(KT / 1024 == lanes::fp8_k_loads(D) &&
                      KT / 1024 == lanes::fp8_v_loads(D),
                  "tile loads");
    toffs[m] = u2 < KT / 1024 ? lanes::fp8_k_src(D, u2, lane)
                              : lanes::fp8_v_src(u2 - KT / 1024, lane);
  }
  const size_t kvh = (size_t)(b * p.Hkv + hk) * p.Nkp * D;
  const miattn_i32x4 krs = rows_rsrc(p.k8 + kvh, p.Nkp * D);
  const miattn_i32x4 vrs = rows_rsrc(p.v8t + kvh, p.Nkp * D);
  // Wave w issues loads w + NW m: the K tile's KL loads split evenly over
  // the waves, so a wave's first KL / NW loads are K and the rest V^T, the
  // same m for every wave (no test per load)
  constexpr int KL = KT / 1024;
  static_assert(KL % NW == 0 && LOADS == LW * NW, "even split of the loads");
  auto issue_k = [&](auto slot_c, int tile) {
    const unsigned tb = (unsigned)(tile * KT);
#pragma unroll
    for (int m = 0; m < KL / NW; ++m) {
      const int u2 = wave + NW * m;
      miattn_buffer_load_lds(krs, (lds_void*)(kslot(slot_c) + u2 * 1024), 16,
                             toffs[m] + tb, 0, 0, 0);
    }
  };
  auto issue_v = [&](auto slot_c, int tile) {
    const unsigned tb = (unsigned)(tile * KT);
#pragma unroll
    for (int m = KL / NW; m < LW; ++m) {
      const int u2 = wave + NW * m;
      miattn_buffer_load_lds(vrs,
                             (lds_void*)(vslot(slot_c) + (u2 - KL) * 1024), 16,
                             toffs[m] + tb, 0, 0, 0);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float M = -INFINITY;  // running maximum (log2 units)
  float l = 0.f;        // this lane's half of the running sum
  const f32x16 zero = {};

  // S^T of tile t (raw accumulators; the score is acc * crow * sk_t)
  auto qk = [&](auto slot_c, f32x16(&s2)[2]) {
    const uint8_t* Kt = kslot(slot_c);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(Kt + koff[mb][ks][0]);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(Kt + koff[mb][ks][1]);
        i32x8 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (int)a0[e];
          a[4 + e] = (int)a1[e];
        }
        s2[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a, qf[ks], ks == 0 ? zero : s2[mb], 0, 0, 0, 127, 0, 127);
      }
  };

  // softmax of tile t on its raw scores sc (skt, svt: the tile's K and V
  // scales): W = P * vr as E4M3 in wb (bytes 0..15: keys 16g + r, 16..31:
  // keys 32 + 16g + r), row sums in l
  auto softmax = [&](auto full_c, int t, f32x16(&sc)[2], i32x8& wb, float skt,
                     float svt) {
    const float cs = crow * skt;
    if (!decltype(full_c)::value && !tile_full(t)) {
      const int j0 = t * kBlk;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = j0 + mb * 32 + 16 * g + r;
          const bool off = (jj >= rk.hc) |
                           (((jj < rk.lo) | (jj >= rk.hw)) & (jj >= rk.sk));
          sc[mb][r] = off ? -INFINITY : sc[mb][r];
        }
    }
    float mr = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mr = fmaxf(mr, sc[mb][r]);
    mr = half_swap_max(mr);
    const float mx = mr * cs;  // cs > 0: the largest score of the row
    if (__builtin_amdgcn_ballot_w64(mx > M + kTau) != 0) {
      const float mn = fmaxf(M, mx);
      const float alpha =
          (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      M = mn;
    }
    // w = 2^(acc cs - M) * vr = 2^(acc cs + (log2 vr - M)); the V ratio is
    // kept above 2^-100 so that a tile of zero V still counts in l
    const float vr = fmaxf(svt * inv_svm, 0x1p-100f);
    const float lv = __builtin_amdgcn_logf(vr) - ((M == -INFINITY) ? 0.f : M);
    float ls = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] = __builtin_amdgcn_exp2f(fmaf(sc[mb][r + e], cs, lv));
          ls += w[e];
        }
        unsigned u = __builtin_amdgcn_cvt_pk_fp8_f32(w[0], w[1], 0u, false);
        u = __builtin_amdgcn_cvt_pk_fp8_f32(w[2], w[3], u, true);
        wb[mb * 4 + r / 4] = (int)u;
      }
    l += ls * __builtin_amdgcn_rcpf(vr);  // 1 ulp; vr in [2^-100, 1]
  };

  // O^T += V^T W^T over tile t's keys
  auto pv = [&](auto slot_c, const i32x8& wb) {
    const uint8_t* Vt = vslot(slot_c);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(Vt + voff[db][0]);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(Vt + voff[db][1]);
      i32x8 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = (int)a0[e];
        a[4 + e] = (int)a1[e];
      }
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          a, wb, oacc[db], 0, 0, 0, 127, 0, 127);
    }
  };

  // Step t: loads of K(t+2) and V(t+1) go out; the S^T product of tile t+1
  // runs on the matrix cores while the softmax of tile t (whose S^T the
  // previous step formed) runs on the vector units; then O^T += V^T W^T of
  // tile t.  K(t) and V(t) live in slot t % 2.
  // Prologue: K(0), V(0), K(1) resident, S^T(0) formed.
  f32x16 sa[2], sb[2];
  if (nt > 0) {
    // the scales of tile t + 1 are read in step t ahead of its tile loads:
    // the wait for them is the end-of-step wait, not one in the softmax
    // behind the loads in flight
    float skc = skh[tile_of(0)], svc = svh[tile_of(0)];
    issue_k(ic<0>(), tile_of(0));
    issue_v(ic<0>(), tile_of(0));
    if (1 < nt) issue_k(ic<1>(), tile_of(1));
    wait_vm0();
    barrier_nofence();
    if (wave_needs(tile_of(0))) qk(ic<0>(), sa);
    auto step = [&](auto par_c, int t, f32x16(&sc)[2], f32x16(&sn)[2]) {
      constexpr int P = decltype(par_c)::value;
      const float skt = skc, svt = svc;
      if (t + 1 < nt) {
        skc = skh[tile_of(t + 1)];
        svc = svh[tile_of(t + 1)];
      }
      if (t + 2 < nt) issue_k(ic<P>(), tile_of(t + 2));
      if (t + 1 < nt) issue_v(ic<1 - P>(), tile_of(t + 1));
      const int tt = tile_of(t);
      const bool need = wave_needs(tt);
      if (t + 1 < nt && wave_needs(tile_of(t + 1))) qk(ic<1 - P>(), sn);
      if (need) {
        i32x8 wb;
        softmax(ic<0>(), tt, sc, wb, skt, svt);
        pv(ic<P>(), wb);
      }
      wait_vm0();
      barrier_nofence();
    };
    // Interior steps [la, lb) of the longer run (the window run when there
    // are two): tiles t and t + 1 are wholly allowed for every row of the
    // wave and the tiles loaded in the step belong to the run.  Such a step
    // is the one above with every decision known: tile t + toff, no mask
    // test, no tests on the loads and the next tile's product.
    int la = 0, lb = 0;
    const int s0 = nt > nA ? nA : 0, s1 = nt > nA ? nt : nA;
    const int toff = nt > nA ? tB0 - nA : 0;
    if (wlive) {
      const int f0 = (wl.lo + kBlk - 1) / kBlk;  // first tile left-full
      const int f1 = wf.hw / kBlk;               // tiles below: right-full
      la = max(s0, f0 - toff);
      lb = min(s1 - 2, f1 - toff - 1);
    }
    auto lean = [&](auto par_c, int t, f32x16(&sc)[2], f32x16(&sn)[2]) {
      constexpr int P = decltype(par_c)::value;
      const float skt = skc, svt = svc;
      skc = skh[t + 1 + toff];
      svc = svh[t + 1 + toff];
      issue_k(ic<P>(), t + 2 + toff);
      issue_v(ic<1 - P>(), t + 1 + toff);
      qk(ic<1 - P>(), sn);
      i32x8 wb;
      softmax(ic<1>(), t + toff, sc, wb, skt, svt);
      pv(ic<P>(), wb);
      wait_vm0();
      barrier_nofence();
    };
    // The loop leaves from inside the pair rather than skipping its second
    // step: the score buffers are dead after the loop, so the swap of roles
    // costs no register copies at a join.  The lean pairs run in a loop of
    // their own, between the general steps before and after them.
    const int lp0 = la + (la & 1);
    const int lp1 = lp0 + 1 < lb ? lp0 + ((lb - lp0) & ~1) : lp0;
    int t = 0;
    for (; t < (lp1 > lp0 ? lp0 : nt); t += 2) {
      step(ic<0>(), t, sa, sb);
      if (t + 1 >= nt) break;
      step(ic<1>(), t + 1, sb, sa);
    }
    if (lp1 > lp0) {
      for (; t < lp1; t += 2) {
        lean(ic<0>(), t, sa, sb);
        lean(ic<1>(), t + 1, sb, sa);
      }
      for (; t < nt; t += 2) {
        step(ic<0>(), t, sa, sb);
        if (t + 1 >= nt) break;
        step(ic<1>(), t + 1, sb, sa);
      }
    }
  }

  // O = O^T * sv_max / 256 / l, lse = (M + log2 l) ln 2
  const float lt = l + __shfl_xor(l, 32);
  if (qi < p.Nq) {
    const bool any = qlive && lt > 0.f;
    const float f = any ? svm / (kPScale * lt) : 0.f;
    uint16_t* orow = p.o + (bhq * p.Nq + qi) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int quad = 0; quad < 4; ++quad) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = oacc[db][4 * quad + e] * f;
        *reinterpret_cast<bf16x4*>(orow + db * 32 + quad * 8 + 4 * g) =
            __builtin_convertvector(v4, bf16x4);
      }
    if (g == 0 && p.lse)
      p.lse[bhq * p.Nq + qi] =
          any ? (M + log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
  if (blockIdx.x >= p.tail.first && threadIdx.x == 0)
    tail_clear(p.tail, tail_done);
}

template <int D>
hipError_t quant_one(QuantParams q, hipStream_t st) {
  const int grid = q.B * q.H * q.nblk;
  QuantSet set = {};
  set.t[0] = q;
  set.first[1] = set.first[2] = set.first[3] = grid;
  set.t[0].mode = 1;
  hipLaunchKernelGGL((fp8_quant_kernel<D>), dim3(grid), dim3(256), 0, st, set);
  hipLaunchKernelGGL(fp8_tensor_amax_kernel, dim3(1), dim3(256), 0, st,
                     q.scales, grid);
  set.t[0].mode = 2;
  hipLaunchKernelGGL((fp8_quant_kernel<D>), dim3(grid), dim3(256), 0, st, set);
  return hipGetLastError();
}

// Block scales: Q, K and V in one launch.
template <int D>
hipError_t quant_three(const QuantParams& a, const QuantParams& k,
                       const QuantParams& v, hipStream_t st) {
  QuantSet set = {};
  set.t[0] = a;
  set.t[1] = k;
  set.t[2] = v;
  set.first[0] = 0;
  set.first[1] = a.B * a.H * a.nblk;
  set.first[2] = set.first[1] + k.B * k.H * k.nblk;
  set.first[3] = set.first[2] + v.B * v.H * v.nblk;
  for (int i = 0; i < 3; ++i) set.t[i].mode = 0;
  hipLaunchKernelGGL((fp8_quant_kernel<D>), dim3(set.first[3]), dim3(256), 0,
                     st, set);
  return hipGetLastError();
}

}  // namespace fp8_impl

using namespace fp8_impl;

hipError_t launch_fp8_quantize(const void* q, const void* k, const void* v,
                               const Problem& pr, const signed char* signs,
                               int per_tensor, void* q8, float* sq, void* k8,
                               float* sk, void* v8t, float* sv,
                               hipStream_t stream) {
  const int nkp = (pr.Nk + kBlk - 1) / kBlk * kBlk;
  QuantParams base = {};
  base.seqlens = pr.seqlens;
  base.B = pr.B;
  base.Nq = pr.Nq;
  base.Nk = pr.Nk;
  base.d = pr.d;
  QuantParams a = base;  // Q
  a.x = static_cast<const uint16_t*>(q);
  a.codes = static_cast<uint8_t*>(q8);
  a.scales = sq;
  a.signs = signs;
  a.H = pr.Hq;
  a.N = pr.Nq;
  a.is_q = 1;
  a.transposed = 0;
  a.Npad = pr.Nq;
  a.nblk = (pr.Nq + kBlk - 1) / kBlk;
  QuantParams bk = base;  // K
  bk.x = static_cast<const uint16_t*>(k);
  bk.codes = static_cast<uint8_t*>(k8);
  bk.scales = sk;
  bk.signs = signs;
  bk.H = pr.Hkv;
  bk.N = pr.Nk;
  bk.is_q = 0;
  bk.transposed = 0;
  bk.Npad = nkp;
  bk.nblk = nkp / kBlk;
  QuantParams c = bk;  // V: never rotated, tiles transposed
  c.x = static_cast<const uint16_t*>(v);
  c.codes = static_cast<uint8_t*>(v8t);
  c.scales = sv;
  c.signs = nullptr;
  c.transposed = 1;
  hipError_t e;
  if (!per_tensor)
    return pr.d == 128 ? quant_three<128>(a, bk, c, stream)
                       : quant_three<64>(a, bk, c, stream);
  if (pr.d == 128) {
    if ((e = quant_one<128>(a, stream)) != hipSuccess) return e;
    if ((e = quant_one<128>(bk, stream)) != hipSuccess) return e;
    return quant_one<128>(c, stream);
  }
  if ((e = quant_one<64>(a, stream)) != hipSuccess) return e;
  if ((e = quant_one<64>(bk, stream)) != hipSuccess) return e;
  return quant_one<64>(c, stream);
}

hipError_t launch_fwd_fp8(const void* q8, const float* sq, const void* k8,
                          const float* sk, const void* v8t, const float* sv,
                          void* o, float* lse, const Problem& pr, int rotated,
                          hipStream_t stream) {
  Fp8Params p;
  p.q8 = static_cast<const uint8_t*>(q8);
  p.sq = sq;
  p.k8 = static_cast<const uint8_t*>(k8);
  p.sk = sk;
  p.v8t = static_cast<const uint8_t*>(v8t);
  p.sv = sv;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.seqlens = pr.seqlens;
  p.B = pr.B;
  p.Hq = pr.Hq;
  p.Hkv = pr.Hkv;
  p.Nq = pr.Nq;
  p.Nk = pr.Nk;
  p.Nkp = (pr.Nk + kBlk - 1) / kBlk * kBlk;
  p.G = pr.Hq / pr.Hkv;
  p.causal = pr.causal;
  p.window = pr.window;
  p.window_right = pr.window_right;
  p.sinks = pr.sinks;
  p.c = fabsf(pr.scale) * 1.4426950408889634f /
        (rotated ? (float)pr.d : 1.0f);
  p.qsign = pr.scale < 0.f ? 0x80808080u : 0u;
  constexpr int NW = 4;
  static_assert(NW == lanes::kFp8Waves, "shared lane layout");
  p.nqb = (pr.Nq + kWR * NW - 1) / (kWR * NW);
  p.total = pr.B * pr.Hq * p.nqb;
  // K and V^T codes of one group: 2 Nkp d bytes; two workgroups per CU
  p.order = make_block_order(pr.B, pr.Hkv, p.G, p.nqb, pr.causal != 0,
                             2LL * p.Nkp * pr.d, 32 * 2);
  // the run-time tail: causal longest-first order with no left window or
  // sinks (so that the last blocks are the light ones)
  int grid = p.total;
  p.tail = make_tail_queue(p.total, 32 * 2, 3,
                           p.order.lpt && p.order.causal && pr.window == 0 &&
                               pr.sinks == 0,
                           &grid);
  if (pr.d == 128)
    hipLaunchKernelGGL((attn_fp8_kernel<128, NW>), dim3(grid),
                       dim3(64 * NW), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fp8_kernel<64, NW>), dim3(grid),
                       dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

}  // namespace miattn
