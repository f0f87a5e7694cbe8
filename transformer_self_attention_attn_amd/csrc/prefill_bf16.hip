// Tiled bf16 attention on gfx950 matrix cores for Nq > 1 query rows: the
// square prefill (Nq == Nk) and a chunk of Nq < Nk new rows against a key/value
// cache or an encoder output (cross-attention, no causal mask).
//
// What is computed: for every (batch b, query head h, live query row i)
//   s_ij = scale * q_i . k_j            (K/V head h / G, allowed keys j only)
//   o_i  = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i)
//   lse_i = m_i + ln sum_j exp(s_ij - m_i)
// i.e. Softmax(Q K^T / sqrt(D)) V of the SpAtten review page (Background -
// Attention Mechanism) with the padding and look-ahead masks of the
// self-attention explainer page and the one-sided local window of the O(n^2)
// tutorial page.  Like the FlashAttention kernels described on the
// FlashAttention-3 review page (FA1/FA2 comparison: one fused kernel, Q/K/V
// cut into on-chip blocks, softmax statistics kept instead of the N x N
// matrix), the scores never leave registers; the design below is this
// library's own, laid out for CDNA4 wave64 MFMA and LDS.
//
// Work decomposition
//   workgroup = NW wavefronts; wave w owns 32 query rows q0 + 32w .. +31 of
//   one head.  The K/V tile loop walks 64-key tiles that at least one row of
//   the workgroup may see (tiles entirely above the causal diagonal, left of
//   the window or past the valid length are never loaded); a wave skips the
//   arithmetic of tiles that none of its rows may see, and only tiles that
//   are partly allowed pay for per-element masking.  The steps in which a
//   wave needs all of a tile and both tiles it loads are whole run in a loop
//   of their own, with every one of these decisions known (no per-step
//   test).  Query heads of one K/V head are adjacent in the launch order and
//   the block index is remapped so that each XCD (own L2) runs whole (batch,
//   K/V head) groups, causal blocks heaviest first (block_order.h).
//
// Data movement
//   K and V tiles go from HBM straight into LDS with 16-byte direct-to-LDS
//   buffer loads (no register staging) into rings of two K and two V
//   slots, each wave issuing its share of a tile's loads.  Each tile is read
//   through a buffer resource that starts at the tile and ends at the valid
//   length, so rows past it read as zeros (padded contents never enter LDS)
//   and a lane's offset within a tile is a constant: issuing a load costs
//   scalar work only.  LDS rows are padded (K: +16 B, V: +64 B per
//   row); with those strides every matrix-operand read below touches each LDS
//   bank once, and every operand address is a per-lane base plus a
//   compile-time offset.  K rows are stored in the order the 32x32 MFMA wants
//   (see k_row_key); V keeps its natural [key][d] order and is read with the
//   transposing LDS read ds_read_b64_tr_b16, which hands each lane four
//   consecutive keys of one column, exactly the A operand of V^T.
//   Ring slots are compile-time constants in every unrolled step, so the
//   compiler can tell the slot being filled from the slots being read and
//   does not stall reads on loads in flight; completion of the tiles needed
//   next is awaited with an explicit wait on outstanding loads, followed by a
//   plain workgroup barrier.
//
// Per tile, per wave (the transposed formulation keeps each query's softmax
// statistics inside one lane pair):
//   S^T[key][query] = K_tile . Q^T     v_mfma_f32_32x32x16_bf16, A = K rows
//                                      from LDS, B = Q^T held in registers
//   online softmax in base 2 (scale * log2 e folded into one FMA); the
//   running maximum is only moved (and O rescaled) when some row's new
//   maximum exceeds it by more than 2^8, which is exact arithmetic: the
//   stored maximum is any common shift of the row's scores
//   O^T[d][query] += V^T . P^T         A = V^T via transposing LDS reads,
//                                      B = P^T (bf16) converted from the
//                                      S^T accumulator
// Two-stage software pipeline: X(t) issues the S^T product of tile t+1 to the
// matrix cores interleaved with the exponentials of tile t (and the tile
// loads), Y(t) the V^T P^T product of tile t interleaved with the bf16
// conversion and row sum of tile t and the maximum of tile t+1.  Two
// workgroups share each CU (LDS and registers are sized for it), so every
// SIMD runs wavefronts of two workgroups whose barriers are independent: they
// drift apart and one wave's X overlaps the other's Y without any offset
// imposed inside a workgroup (three workgroups per CU at d = 64).
#include "kernels.h"

#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "block_order.h"
#include "tail_queue.h"

// Workgroup shape per head dimension, chosen by measurement on MI355X: both
// run 4 wavefronts (128 query rows share each K/V tile) with at least two
// workgroups per CU.  At d=128 one workgroup of 8 wavefronts per CU, its two
// halves offset by half a tile, was 3-6% slower.
#ifndef MIATTN_PREFILL_NW128
#define MIATTN_PREFILL_NW128 4
#endif
#ifndef MIATTN_PREFILL_NW64
#define MIATTN_PREFILL_NW64 4
#endif

namespace miattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kQW = 32;          // query rows per wavefront
constexpr int kKT = 64;          // keys per tile
constexpr float kTau = 8.0f;     // lazy-rescale threshold, log2 units

template <int D, int NW>
struct Cfg {
  static constexpr int THREADS = 64 * NW;
  static constexpr int QB = kQW * NW;    // query rows per workgroup
  static constexpr int KSTR = D + 8;     // K tile row stride (elements)
  static constexpr int VSTR = D + 32;    // V tile row stride (elements)
  static constexpr int KSLOTS = KSTR / 8;  // 16-byte slots per K row
  static constexpr int VSLOTS = VSTR / 8;
  static constexpr int KTILE = kKT * KSTR;
  static constexpr int VTILE = kKT * VSTR;
  static constexpr int KLOADS = kKT * KSLOTS / 64;  // wave-wide 1 KB loads
  static constexpr int VLOADS = kKT * VSLOTS / 64;
  static constexpr int KLW = (KLOADS + NW - 1) / NW;  // per wave, at most
  static constexpr int VLW = (VLOADS + NW - 1) / NW;
  static constexpr int KS = D / 16;  // k-steps of the S^T product
  static constexpr int DB = D / 32;  // 32-row blocks of O^T
  static_assert(kKT * KSLOTS % 64 == 0 && kKT * VSLOTS % 64 == 0, "split");
  static_assert(KSLOTS == lanes::prefill_k_chunks(D) &&
                    VSLOTS == lanes::prefill_v_chunks(D) &&
                    KLOADS == lanes::prefill_k_loads(D) &&
                    VLOADS == lanes::prefill_v_loads(D) &&
                    NW == lanes::kPrefillWaves && kKT == lanes::kTileRows,
                "tile loads as the shared lane layout states them");
  static_assert(KLW + VLW <= 4 * DB, "interleaved loads fit the PV product");
  // two workgroups per CU: K and V rings and the 1 KB load sink of each fit
  // in half of the 160 KB of LDS
  static_assert((2 * KTILE + 2 * VTILE) * 2 + 1024 <= 80 * 1024, "LDS");
};

// Key held in row r of the K tile in LDS.  Rows are in MFMA row order: with
// this order the 32x32 accumulator of S^T gives lane group g (lanes 32g ..
// 32g+31) the 16 consecutive keys g*16 .. g*16+15 of each 32-key block.
__device__ inline int k_row_key(int r) { return lanes::mfma_row(r); }

// Waits until at most n vector-memory loads of this wave are outstanding
// (the direct-to-LDS loads count there); the other counters are left alone.
__device__ inline void wait_vmcnt(int n) {
#define MIATTN_VM(N)                                                      \
  case N:                                                                 \
    __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | 0xF70); \
    break;
  switch (n) {
    MIATTN_VM(0) MIATTN_VM(1) MIATTN_VM(2) MIATTN_VM(3) MIATTN_VM(4)
    MIATTN_VM(5) MIATTN_VM(6) MIATTN_VM(7) MIATTN_VM(8) MIATTN_VM(9)
    MIATTN_VM(10) MIATTN_VM(11) MIATTN_VM(12) MIATTN_VM(13) MIATTN_VM(14)
    MIATTN_VM(15) MIATTN_VM(16) MIATTN_VM(17) MIATTN_VM(18) MIATTN_VM(19)
    MIATTN_VM(20) MIATTN_VM(21) MIATTN_VM(22) MIATTN_VM(23) MIATTN_VM(24)
    default:
      __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  }
#undef MIATTN_VM
}

// Workgroup barrier without a memory fence: every LDS read of a tile is
// consumed within the tile, and the loads the next tile needs were awaited
// with wait_vmcnt.  The clobber keeps the compiler from moving memory
// accesses across it.
__device__ inline void barrier_nofence() {
  asm volatile("s_barrier" ::: "memory");
}

// max(x, x of the lane 32 apart), on the VALU: v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second;
// both start as x, so afterwards one holds x of the lower half and the other
// x of the upper half in every lane.  Written as inline assembly with two
// distinct registers: the builtin given the same value twice was folded to
// a single result.
// The maximum is taken inside the same block, so the compiler does not
// canonicalize the two swapped values before it (they are never NaN).
__device__ inline float half_swap_max(float x) {
  float a = x, b = x;
  asm volatile(
      "s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(a), "+v"(b));
  return a;
}

// x of this lane plus x of the lane 32 away, the same way
__device__ inline float half_swap_add(float x) {
  float a = x, b = x;
  asm volatile(
      "s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\t"
      "v_add_f32 %0, %0, %1"
      : "+v"(a), "+v"(b));
  return a;
}

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* seqlens;
  int B, Hq, Hkv, Nq, Nk, G, nqb, causal, window, window_right, sinks, total;
  float c;         // |scale| * log2(e) (a tiny positive value for scale 0)
  unsigned qsign;  // 0x80008000 when scale < 0: Q is negated on load
  BlockOrder order;  // block -> (batch, head, query block): block_order.h
  TailQueue tail;    // lightest blocks handed out at run time: tail_queue.h
};

template <int I>
using ic = std::integral_constant<int, I>;

// Mask kinds, one kernel each so that the masked tile's code has one path
// (a run-time choice among three made the compiler copy every score at the
// join): keys below a right limit only (look-ahead, padding, right window),
// a left window as well, and attention sinks as well.
enum MaskKind { kMaskRight = 0, kMaskWindow = 1, kMaskSinks = 2 };

template <int D, int NW, int MK>
__global__ __launch_bounds__(64 * NW, D == 64 ? 3 : 2) void prefill_kernel(
    PrefillParams p) {
  using C = Cfg<D, NW>;
  // the left window and the sink count, 0 where the kind has none
  const int window = MK == kMaskRight ? 0 : p.window;
  const int sinks = MK == kMaskSinks ? p.sinks : 0;
  // one LDS object per ring slot: the compiler keeps per-object alias
  // scopes, which lets reads of one slot proceed while another is filled
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[C::KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[C::KTILE];

  __shared__ __attribute__((aligned(16))) uint16_t Vs0[C::VTILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[C::VTILE];
  auto kslot = [&](auto s_c) -> uint16_t* {
    constexpr int S = decltype(s_c)::value;
    if constexpr (S == 0) return Ks0;
    else return Ks1;
  };
  auto vslot = [&](auto s_c) -> uint16_t* {
    constexpr int S = decltype(s_c)::value;
    if constexpr (S == 0) return Vs0;
    else return Vs1;
  };

  // ---- block -> (batch, head, query block) --------------------------------
  // the order of block_order.h: whole (batch, K/V head) groups per XCD,
  // causal blocks heaviest first; from p.tail.first on, the workgroups take
  // the lightest blocks from the run-time queue of tail_queue.h
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

  int L = p.Nk;
  if (p.seqlens) {
    L = p.seqlens[b];
    L = L < 0 ? 0 : (L > p.Nk ? p.Nk : L);
  }
  // Nq == Nk: the first L rows are live and row i sits at position i.
  // Nq != Nk: all Nq rows are live and are the last Nq positions of the
  // sequence, row i at position L - Nq + i (negative when L < Nq: such a row
  // sees no key under the causal mask).
  const int Lq = (p.Nq == p.Nk) ? L : p.Nq;
  const int off = L - Lq;

  const int tid = threadIdx.x;
  // wave index as a scalar: load numbers and LDS destinations derived from
  // it stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int q0 = qb * C::QB;
  const int qw0 = q0 + wave * kQW;
  const int qi = qw0 + ql;

  const size_t qo_base = (size_t)(b * p.Hq + h) * p.Nq * D;
  const size_t kv_base = (size_t)(b * p.Hkv + hk) * p.Nk * D;
  const uint16_t* kg = p.k + kv_base;
  const uint16_t* vg = p.v + kv_base;

  // ---- key ranges ---------------------------------------------------------
  // Row qi at position pos may see keys below hc (the valid length, and
  // pos + 1 under the causal mask); of those, the window keys lo <= j < hw
  // (left limit pos - j < window, right limit j - pos < window_right, each
  // off when 0) and the sink keys j < sk.  Every bound is 0 on a dead row.
  const bool qlive = qi < Lq;
  const int pos = qi + off;
  auto cap = [&](int rpos) {  // hc of the row at position rpos
    return max(0, p.causal ? min(L, rpos + 1) : L);
  };
  auto right = [&](int rpos, int h) {  // hw of that row, given hc = h
    return p.window_right > 0 ? max(0, min(h, rpos + p.window_right)) : h;
  };
  auto left = [&](int rpos) {
    return window > 0 ? max(0, rpos - window + 1) : 0;
  };
  const int hc = qlive ? cap(pos) : 0;
  const int hw = right(pos, hc);
  const int lo = qlive ? left(pos) : 0;
  const int sk = min(sinks, hc);

  // Tiles the workgroup visits: the sink tiles [0, ts1), then the window
  // tiles [tw0, tw1) (merged into one run when they meet).  Step k of the
  // loop visits tile tile_of(k), k in [0, nt).
  const int rows_end = min(q0 + C::QB, Lq);
  int nA = 0, tB0 = 0, nt = 0;
  if (rows_end > q0) {
    const int pl = rows_end - 1 + off;  // position of the last live row
    const int kv_hc = cap(pl);
    const int kv_hi = right(pl, kv_hc);
    const int kv_lo = left(q0 + off);
    int tw0 = kv_lo / kKT, tw1 = (kv_hi + kKT - 1) / kKT;
    if (kv_hi <= kv_lo) tw0 = tw1 = 0;
    const int ts1 = (min(sinks, kv_hc) + kKT - 1) / kKT;
    if (ts1 >= tw0) {
      nA = max(ts1, tw1);
      nt = nA;
    } else {
      nA = ts1;
      tB0 = tw0;
      nt = ts1 + (tw1 - tw0);
    }
  }
  auto tile_of = [&](int k) { return k < nA ? k : tB0 + (k - nA); };

  // the same bounds over the wave's live rows qw0 .. wend-1: their union
  // (wave_needs) and their intersection (tile_full: no mask needed)
  const int wend = min(qw0 + kQW, Lq);
  const bool wlive = wend > qw0;
  const int wpf = qw0 + off, wpl = wend - 1 + off;
  const int w_hc_max = cap(wpl), w_hc_min = cap(wpf);
  const int w_hi_max = right(wpl, w_hc_max);
  const int w_hi_min = right(wpf, w_hc_min);
  const int w_lo_min = left(wpf), w_lo_max = left(wpl);
  const int w_sk_max = min(sinks, w_hc_max);
  const int w_sk_min = min(sinks, w_hc_min);
  auto wave_needs = [&](int t) {
    const int j0 = t * kKT;
    return wlive &&
           ((j0 < w_hi_max && j0 + kKT > w_lo_min) || j0 < w_sk_max);
  };
  auto tile_full = [&](int t) {
    const int j0 = t * kKT;
    return (j0 >= w_lo_max && j0 + kKT <= w_hi_min) || j0 + kKT <= w_sk_min;
  };

  // ---- Q^T fragments (B operand), kept in registers -----------------------
  // Read through a resource that ends at the live rows (Lq rows of the
  // head): a dead row reads as zeros, with no branch per load.  The sign of
  // a negative scale is applied just before the first product, so that
  // nothing waits for these loads before then.
  bf16x8 qf[C::KS];
  {
    const miattn_i32x4 qrs = dev::rows_rsrc(p.q + qo_base, Lq * D * 2);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qf[ks] = __builtin_bit_cast(
          bf16x8, miattn_buffer_load_b128(qrs, (qi * D + 16 * ks + 8 * g) * 2,
                                          0, 0));
  }

  // ---- direct-to-LDS tile loads ---------------------------------------------
  // Wave-wide load i fills LDS bytes [i * 1024, +1024) of the tile: lane l
  // writes 16-byte slot i*64 + l, i.e. (row, chunk) of the padded row.  Loads
  // are dealt round-robin to the waves; each lane's byte offset within a
  // tile is fixed, so it is computed once.  Pad chunks are never read and
  // take the row's first chunk.  A tile is read through a buffer resource
  // that starts at the tile and ends at the valid length: rows past it read
  // as zeros, so padded contents never enter LDS.
  unsigned kvo[C::KLW], vvo[C::VLW];
#pragma unroll
  for (int m = 0; m < C::KLW; ++m)
    kvo[m] = lanes::prefill_k_src(D, wave + NW * m, lane);
#pragma unroll
  for (int m = 0; m < C::VLW; ++m)
    vvo[m] = lanes::prefill_v_src(D, wave + NW * m, lane);
  // resource of tile t of K or V (`live`: a tile of the plan; otherwise an
  // empty range, whose reads touch no memory)
  auto tile_rsrc = [&](const uint16_t* base, int t, bool live) {
    return dev::rows_rsrc(live ? base + (size_t)t * kKT * D : base,
                          lanes::prefill_tile_bytes(D, L, t, live));
  };
  // Interleaved loads (issued during X): every wave issues KLW + VLW of
  // them per tile.  A wave without a load number m (uneven split) writes
  // into a 1 KB sink instead of the slot; a step with no tile to load reads
  // through an empty resource, whose zeros land in a slot nothing reads
  // before it is loaded again.
  __shared__ __attribute__((aligned(16))) uint16_t Sink[512];
  auto dma_il = [&](miattn_i32x4 rs, uint16_t* slot, unsigned vo, int i,
                    int nloads) {
    miattn_buffer_load_lds(rs, (lds_void*)(i < nloads ? slot + i * 512 : Sink),
                           16, (int)vo, 0, 0, 0);
  };

  auto dma_k = [&](auto slot_c, int t) {
    const miattn_i32x4 rs = tile_rsrc(kg, t, true);
#pragma unroll
    for (int m = 0; m < C::KLW; ++m) {
      const int i = wave + NW * m;
      // (only a load number past NW (m + 1) can be out of range)
      if (NW * (m + 1) <= C::KLOADS || i < C::KLOADS)
        miattn_buffer_load_lds(rs, (lds_void*)(kslot(slot_c) + i * 512), 16,
                               (int)kvo[m], 0, 0, 0);
    }
  };
  auto dma_v = [&](auto slot_c, int t) {
    const miattn_i32x4 rs = tile_rsrc(vg, t, true);
#pragma unroll
    for (int m = 0; m < C::VLW; ++m) {
      const int i = wave + NW * m;
      if (NW * (m + 1) <= C::VLOADS || i < C::VLOADS)
        miattn_buffer_load_lds(rs, (lds_void*)(vslot(slot_c) + i * 512), 16,
                               (int)vvo[m], 0, 0, 0);
    }
  };

  // ---- S^T = K . Q^T for one tile (no interleaving) -----------------------
  auto qk = [&](auto slot_c, f32x16(&s)[2]) {
    constexpr int S = decltype(slot_c)::value;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const uint16_t* kr = kslot(slot_c) + (mb * 32 + ql) * C::KSTR + 8 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 16 * ks);
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0,
                                                        0);
      }
    }
  };

  // V^T operand: lane i of 16-lane group G reads, for 4 keys at a time, the
  // column dbase + i; source lane s addresses row key0 + s/4, columns
  // dbase + 4*(s%4) .. +3.
  const int grp16 = lane >> 4;
  const int i16 = lane & 15;
  const int v_lane = (i16 >> 2) * C::VSTR + 16 * (grp16 & 1) + 4 * (i16 & 3);

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float M = -INFINITY;  // running maximum of s * c (log2 units)
  float l = 0.f;        // this lane's half of the running sum

  float mx_pre = -INFINITY;
  // One tile of work for a wave, on the scores `sc` of tile t (V slot SV);
  // the S^T product of tile t+1 (K slot SK) is issued into `sn`, interleaved
  // with this tile's exponentials (at the end of the range it reads a stale
  // slot and the result is dropped).
  // kbi / vbi: tile bases of this step's interleaved K / V loads (into slots
  // SLK / SLV).
  // X(t): mask and maximum of tile t's scores `sc`, lazy rescale, and the
  // S^T product of tile t+1 (K slot SK) into `sn`, interleaved with tile t's
  // exponentials and with this wave's share of a tile load pair (K into slot
  // SLK from resource krs, V into slot SLV from vrs); the weights of tile t
  // stay in
  // `sc` (fp32) for Y(t).
  auto tileX = [&](auto sk_c, auto slk_c, auto slv_c, auto full_c,
                   miattn_i32x4 krs, miattn_i32x4 vrs, int t,
                   f32x16(&sc)[2], f32x16(&sn)[2]) {
    constexpr int SK = decltype(sk_c)::value;
    constexpr bool FULL = decltype(full_c)::value != 0;
    const int j0 = t * kKT;
    float mx = mx_pre;
    // lane holds keys j0 + mb*32 + g*16 + r (r = 0..15) of query qi
    if (!FULL && !tile_full(t)) {
      // this lane's keys of block mb are jb + r, r = 0 .. 15; the bounds are
      // taken relative to jb so that each test compares with a constant r
      if constexpr (MK == kMaskRight) {  // keys below hw only
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int hi = hw - (j0 + mb * 32 + g * 16);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (r >= hi) sc[mb][r] = -INFINITY;
        }
      } else if constexpr (MK == kMaskWindow) {  // keys in [lo, hw)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int jb = j0 + mb * 32 + g * 16;
          const int lor = lo - jb, hi = hw - jb;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (r < lor || r >= hi) sc[mb][r] = -INFINITY;
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + mb * 32 + g * 16 + r;
            if ((j < lo || j >= hw) && j >= sk) sc[mb][r] = -INFINITY;
          }
      }
      mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[mb][r]);
    }
    mx = half_swap_max(mx);
    const float tm = (mx == -INFINITY) ? -INFINITY : mx * p.c;
    const bool need = tm > M + kTau;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float mn = fmaxf(M, tm);
      const float alpha =
          (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      M = mn;
    }
    const float mu = (M == -INFINITY) ? 0.f : M;

    // S^T(t+1) = K(t+1) . Q^T interleaved with this tile's exponentials.
    // K operand reads run four MFMAs ahead of their use.
    constexpr int NQK = 2 * C::KS;  // MFMAs of the S^T product
    constexpr int EPS = 32 / NQK;   // exponentials per MFMA slot
    const uint16_t* kbase = kslot(sk_c) + ql * C::KSTR + 8 * g;
    auto kread = [&](int i) {
      const int mb = i / C::KS, ks = i % C::KS;
      return *reinterpret_cast<const bf16x8*>(kbase + mb * 32 * C::KSTR +
                                              16 * ks);
    };
    bf16x8 ka[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ka[i] = kread(i);
    // keep the first operand reads ahead of the interleaved loop: the
    // scheduler fills the loop's LDS-read slots in program order
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int mb = i / C::KS, ks = i % C::KS;
      if (ks == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[mb][r] = 0.f;
      }
      sn[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i & 3], qf[ks],
                                                       sn[mb], 0, 0, 0);
      if (i + 4 < NQK) ka[i & 3] = kread(i + 4);
      // masked scores are -inf and c > 0, so their weights are exactly 0
#pragma unroll
      for (int u = 0; u < EPS; ++u) {
        const int el = i * EPS + u;
        const int emb = el >> 4, er = el & 15;
        const float e = __builtin_amdgcn_exp2f(fmaf(sc[emb][er], p.c, -mu));
        sc[emb][er] = e;
      }
      // this step's loads, one per MFMA slot
      if (i < C::KLW)
        dma_il(krs, kslot(slk_c), kvo[i], wave + NW * i, C::KLOADS);
      else if (i < C::KLW + C::VLW)
        dma_il(vrs, vslot(slv_c), vvo[i - C::KLW], wave + NW * (i - C::KLW),
               C::VLOADS);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, EPS, 0);      // VALU
      __builtin_amdgcn_sched_group_barrier(0x400, EPS, 0);      // exp
      if (i < C::KLW + C::VLW)
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // load
    }
  };

  // Y(t): O^T += V^T . P^T from V slot SV, interleaved with the bf16
  // conversion and row sum of this tile's weights `sc` and the maximum of
  // the next tile's scores `sn`.
  auto tileY = [&](auto sv_c, const f32x16(&sc)[2], const f32x16(&sn)[2]) {
    // P^T operands (bf16) converted from this tile's weights just ahead of
    // the MFMAs that take them
    auto cvt = [&](int mb, int m) {
      f32x8 pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = sc[mb][8 * m + e];
      return __builtin_convertvector(pv, bf16x8);
    };
    bf16x8 pcur = cvt(0, 0), pnext = pcur;
    // O^T += V^T . P^T; V operand reads run two MFMAs ahead.
    constexpr int NPV = 4 * C::DB;
    auto vread = [&](int i) {
      const int mb = i / (2 * C::DB), m = (i / C::DB) & 1, db = i % C::DB;
      const int key0 = mb * 32 + 16 * g + 8 * m;
      bf16x8 a;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint16_t* ptr =
            vslot(sv_c) + v_lane + (key0 + 4 * half) * C::VSTR + db * 32;
        const i16x4 r4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ptr));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a[4 * half + e] = __builtin_bit_cast(__bf16, (short)r4[e]);
      }
      return a;
    };
    // two partial maxima and sums, each started from its first element
    float mn2[2], l2[2];
    bf16x8 va[5];
#pragma unroll
    for (int i = 0; i < 4; ++i) va[i] = vread(i);
    // keep the first operand reads ahead of the interleaved loop: the
    // scheduler fills the loop's LDS-read slots in program order
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int mb = i / (2 * C::DB), m = (i / C::DB) & 1, db = i % C::DB;
      if (i + 4 < NPV) va[(i + 4) % 5] = vread(i + 4);
      if (db == 0 && i + C::DB < NPV)
        pnext = cvt((i + C::DB) / (2 * C::DB), ((i + C::DB) / C::DB) & 1);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 5], pcur,
                                                         oacc[db], 0, 0, 0);
      // the next tile's maximum, 32 / NPV of its 32 elements per MFMA slot
#pragma unroll
      for (int u = 0; u < 32 / NPV; ++u) {
        const int el = i * (32 / NPV) + u;
        const float x = sn[el >> 4][el & 15];
        mn2[el & 1] = el < 2 ? x : fmaxf(mn2[el & 1], x);
      }
      // the 32 weights of this lane (the row sum in fp32: lse needs the
      // exact sum), 32 / NPV of them per MFMA slot
#pragma unroll
      for (int u = 0; u < 32 / NPV; ++u) {
        const int el = i * (32 / NPV) + u;
        const float x = sc[el >> 4][el & 15];
        l2[el & 1] = el < 2 ? x : l2[el & 1] + x;
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (db == C::DB - 1) pcur = pnext;
    }
    mx_pre = fmaxf(mn2[0], mn2[1]);
    l += l2[0] + l2[1];
  };

  f32x16 sa[2], sb[2];
  // Step t runs X(t) Y(t), then waits for this wave's loads and takes the
  // workgroup barrier.  X(t) reads K(t+1) and loads each wave's share of
  // K(t+2) (over K(t), read by X(t-1)) and V(t+1) (over V(t-1), read by
  // Y(t-1)); Y(t) reads V(t).  K and V of step t (tile tile_of(t)) live in
  // slot t % 2.
  // ---- prologue: K(0), K(1), V(0) resident, S^T(0) formed ----------------
  if (nt > 0) {
    dma_k(ic<0>(), tile_of(0));
    dma_v(ic<0>(), tile_of(0));
    if (1 < nt) dma_k(ic<1>(), tile_of(1));
  }
  if (p.qsign != 0) {  // negative scale: Q negated (uniform branch)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 raw = __builtin_bit_cast(u32x4, qf[ks]);
      raw ^= p.qsign;
      qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  wait_vmcnt(0);
  barrier_nofence();
  if (nt > 0 && wave_needs(tile_of(0))) {
    qk(ic<0>(), sa);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx_pre = fmaxf(mx_pre, sa[mb][r]);
  }
  barrier_nofence();

  auto step = [&](auto k_c, int t, f32x16(&sc)[2], f32x16(&sn)[2]) {
    constexpr int K = decltype(k_c)::value;
    constexpr int SLK = K % 2, SLV = (K + 1) % 2;
    const int tk = t + 2, tv = t + 1;  // steps whose tiles load now
    const int rt = tile_of(t), rk = tile_of(tk), rv = tile_of(tv);
    const bool ld_k = tk < nt, ld_v = tv < nt;
    const bool il = wave_needs(rt);  // this wave's loads go inside X(t)
    if (!il && ld_v) dma_v(ic<SLV>(), rv);
    if (!il && ld_k) dma_k(ic<SLK>(), rk);
    if (il) {
      tileX(ic<(K + 1) % 2>(), ic<SLK>(), ic<SLV>(), ic<0>(),
            tile_rsrc(kg, rk, ld_k), tile_rsrc(vg, rv, ld_v), rt, sc, sn);
    } else if (t + 1 < nt && wave_needs(tile_of(t + 1))) {
      qk(ic<(K + 1) % 2>(), sn);
      mx_pre = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx_pre = fmaxf(mx_pre, sn[mb][r]);
    }
    if (il) tileY(ic<K % 2>(), sc, sn);
    wait_vmcnt(0);
    barrier_nofence();
  };
  // Interior steps [la, lb) of the longer run (the window run when there are
  // two): the wave needs all of the tile with no mask, and the K and V tiles
  // loaded in the step belong to the same run and lie wholly below the valid
  // length.  Such a step is the one above with every decision known: the
  // step works on tile t + toff, its loads read whole 64-row tiles, and no
  // tile bounds are evaluated.  The sink clause of tile_full is left out
  // (fewer lean steps, never a wrong one).
  int la = 0, lb = 0;
  const int s0 = nt > nA ? nA : 0, s1 = nt > nA ? nt : nA;
  const int toff = nt > nA ? tB0 - nA : 0;
  if (wlive) {
    const int f0 = (w_lo_max + kKT - 1) / kKT;  // first tile with no key left of a row's window
    const int f1 = w_hi_min / kKT;              // tiles below: no key right of it
    la = max(s0, f0 - toff);
    lb = min(min(s1 - 2, f1 - toff), L / kKT - 2 - toff);
  }
  const miattn_i32x4 krs0 = dev::rows_rsrc(kg + (size_t)toff * kKT * D, kKT * D * 2);
  const miattn_i32x4 vrs0 = dev::rows_rsrc(vg + (size_t)toff * kKT * D, kKT * D * 2);
  // resource of whole tile t + toff, from the run's base: the 64-bit base
  // advances by whole tiles
  auto lean_rsrc = [&](miattn_i32x4 r0, int t) {
    const unsigned long long a =
        ((unsigned long long)(unsigned)r0[1] << 32 | (unsigned)r0[0]) +
        (unsigned long long)(unsigned)t * (kKT * D * 2);
    miattn_i32x4 r = r0;
    r[0] = (int)(unsigned)a;
    r[1] = (int)((unsigned)(a >> 32) & 0xffffu);
    return r;
  };
  auto lean = [&](auto k_c, int t, f32x16(&sc)[2], f32x16(&sn)[2]) {
    constexpr int K = decltype(k_c)::value;
    constexpr int SLK = K % 2, SLV = (K + 1) % 2;
    tileX(ic<(K + 1) % 2>(), ic<SLK>(), ic<SLV>(), ic<1>(),
          lean_rsrc(krs0, t + 2), lean_rsrc(vrs0, t + 1), t + toff, sc, sn);
    tileY(ic<K % 2>(), sc, sn);
    wait_vmcnt(0);
    barrier_nofence();
  };
  // Unrolled by 2: every ring slot index is a compile-time constant and the
  // two score buffers swap roles without copies (the loop leaves from inside
  // the pair: the buffers are dead after it, so no join needs a copy).
  // The lean pairs start at the first even step from la on.
  const int lp0 = la + (la & 1);
  const int lp1 = lp0 + 1 < lb ? lp0 + ((lb - lp0) & ~1) : lp0;  // end of the pairs
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

  // ---- epilogue -----------------------------------------------------------
  const float lt = half_swap_add(l);
  if (qi < p.Nq) {
    const bool any = qlive && lt > 0.f;
    const float inv = any ? __builtin_amdgcn_rcpf(lt) : 0.f;  // 1 ulp
    uint16_t* orow = p.o + qo_base + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int quad = 0; quad < 4; ++quad) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = oacc[db][4 * quad + e] * inv;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 o4 = __builtin_convertvector(v4, bf16x4);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + quad * 8 + 4 * g) = o4;
      }
    if (g == 0 && p.lse) {
      p.lse[(size_t)(b * p.Hq + h) * p.Nq + qi] =
          any ? (M + log2f(lt)) * 0.69314718055994531f : -INFINITY;
    }
  }
  if (blockIdx.x >= p.tail.first && threadIdx.x == 0)
    tail_clear(p.tail, tail_done);
}

template <int D, int NW, int MK>
void launch(const PrefillParams& p0, hipStream_t stream) {
  using C = Cfg<D, NW>;
  PrefillParams p = p0;
  p.nqb = (p.Nq + C::QB - 1) / C::QB;
  p.total = p.B * p.Hq * p.nqb;
  // bands of the causal block order: with 1 MB of K/V or more per group,
  // the smallest divisor of nqb whose band of one group (qband * G blocks)
  // fills an XCD's workgroup slots (32 CUs); otherwise 1 (plain heaviest
  // first across the XCD's groups)
  constexpr int kSlots = 32 * (D == 64 ? 3 : 2);  // workgroups per XCD at once
  p.order = make_block_order(p.B, p.Hkv, p.G, p.nqb, p.causal != 0,
                             2LL * p.Nk * D * 2, kSlots);
  // the run-time tail: causal longest-first order with no left window (so
  // that the last blocks are the light ones)
  int grid = p.total;
  p.tail = make_tail_queue(p.total, kSlots, 3,
                           p.order.lpt && p.order.causal && MK == kMaskRight,
                           &grid);
  hipLaunchKernelGGL((prefill_kernel<D, NW, MK>), dim3(grid),
                     dim3(C::THREADS), 0, stream, p);
}

}  // namespace

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v,
                               void* o, float* lse, const Problem& pr,
                               hipStream_t stream) {
  PrefillParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.seqlens = pr.seqlens;
  p.B = pr.B;
  p.Hq = pr.Hq;
  p.Hkv = pr.Hkv;
  p.Nq = pr.Nq;
  p.Nk = pr.Nk;
  p.G = pr.Hq / pr.Hkv;
  p.causal = pr.causal;
  p.window = pr.window;
  p.window_right = pr.window_right;
  p.sinks = pr.sinks;
  p.c = fabsf(pr.scale) * 1.4426950408889634f;
  // scale 0: every allowed key weighs the same.  A tiny positive factor keeps
  // masked scores at -inf * c = -inf (weight exactly 0) while every allowed
  // weight 2^(s*c - m) still rounds to exactly 1.0f, as with c = 0.
  if (p.c == 0.f) p.c = 1e-30f;
  p.qsign = (pr.scale < 0.f) ? 0x80008000u : 0u;
  const int mk = p.sinks > 0 ? kMaskSinks : p.window > 0 ? kMaskWindow : kMaskRight;
  if (pr.d == 128) {
    if (mk == kMaskRight) launch<128, MIATTN_PREFILL_NW128, kMaskRight>(p, stream);
    else if (mk == kMaskWindow) launch<128, MIATTN_PREFILL_NW128, kMaskWindow>(p, stream);
    else launch<128, MIATTN_PREFILL_NW128, kMaskSinks>(p, stream);
  } else {
    if (mk == kMaskRight) launch<64, MIATTN_PREFILL_NW64, kMaskRight>(p, stream);
    else if (mk == kMaskWindow) launch<64, MIATTN_PREFILL_NW64, kMaskWindow>(p, stream);
    else launch<64, MIATTN_PREFILL_NW64, kMaskSinks>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace miattn
