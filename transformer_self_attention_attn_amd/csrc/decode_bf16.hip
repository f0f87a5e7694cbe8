// One-token decode attention (Nq == 1), bf16 K/V cache, split over keys.
//
// The generation step processes a single new token whose K and V have been
// appended to the cache (SpAtten review page, Background - Attention-Based NLP
// Models); the page notes this stage is memory-bound.  The query is the last
// token of its sequence: it may see keys j < L_b (and, with a window w, only
// j >= L_b - w; sink keys j < sinks always).
//
// Pass 1 (decode_split_kernel): grid = (batch, K/V head, head chunk) x split,
//   one wavefront per workgroup.  A wavefront owns a chunk of `chunk` keys of
//   one (batch, K/V head) and the (up to 16) query heads of that group that
//   share it, so each K and V byte is read from HBM once for all of them.
//   The heads sharing a K/V head make the step a small matrix product, so it
//   runs on the matrix cores (16 x 16 tiles, heads padded to 16):
//     S^T[key][head] = K_tile . Q^T        v_mfma_f32_16x16x32_bf16
//     O^T[d][head]  += V_tile^T . P^T      v_mfma_f32_16x16x16_bf16
//   K and V stream through a ring of kStages LDS stages (16 keys each, K and
//   V) filled by direct-to-LDS loads issued kStages - 1 tiles ahead; the K
//   operand is read with ds_read_b128 and the V^T operand with the
//   transposing ds_read_b64_tr_b16, both conflict-free under a 16-byte chunk
//   permutation of the tile rows.  Each lane holds 4 keys of one head per
//   tile; the online softmax (base 2, the running maximum moved only when a
//   score exceeds it by more than 2^8) needs one exchange across the 4 lane
//   groups per tile.  The wavefront writes the chunk's partial result
//   o_s = o / l (fp32) and lse_s = (m + log2 l) ln 2 to the workspace.
//   Chunks that hold no allowed key exit at once.
// Pass 2 (decode_combine_kernel): one wavefront per (batch, query head).
//   lse = log sum_s exp(lse_s) (max-shifted) and
//   o = sum_s exp(lse_s - lse) o_s, the softmax definition applied to a
//   partition of the keys; written as bf16 o and fp32 lse.
#include "kernels.h"

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "fastdiv.h"

namespace miattn {
namespace {

using namespace dev;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

#ifndef MIATTN_DECODE_STAGES
#define MIATTN_DECODE_STAGES 4
#endif
// Keys per split: chosen per problem (decode_chunk), a power of two in
// [kMinChunk, kMaxChunk] unless the grid's split limit asks for more.
constexpr int kMinChunk = 128;
constexpr int kMaxChunk = 1024;
constexpr int kMaxSplits = 65535;  // grid y
// Decode wavefronts the chip holds at once: 256 CUs, 5 per CU (LDS-bound).
constexpr long long kSlots = 256 * 5;
constexpr int kStages = MIATTN_DECODE_STAGES;  // LDS ring stages per wave
constexpr int kKT = 16;          // keys per tile
constexpr float kTau = 8.0f;     // lazy-rescale threshold, log2 units
constexpr int kCols = 16;        // query columns per wavefront (MFMA N)
// 1 < Nq < Nk goes to this kernel when its (head, row) columns fill one
// wavefront per K/V head; taller chunks take the prefill kernel (a 32-row
// chunk against 1024 keys, two column blocks, ran 10% slower here)
constexpr int kMaxColumnBlocks = 1;
constexpr int kCombineWaves = 4;  // (batch, head) rows per combine workgroup
constexpr int kNonTemporal = 2;  // cache policy of the K/V loads: streamed

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* seqlens;
  float* ws_o;    // [B, Hq, Nq, nsplit, D]
  float* ws_lse;  // [B, Hq, Nq, nsplit]
  int B, Hq, Hkv, Nq, Nk, G, ncols, nhc, causal, window, window_right, sinks,
      nsplit, chunk;
  float c;  // scale * log2(e)
  // divisions by launch-fixed values (fastdiv.h): Hkv * nhc, nhc, Nq, chunk
  UDiv dv_nx, dv_nhc, dv_nq, dv_chunk;
};

// Valid length of batch b.
__device__ inline int valid_len(const DecodeParams& p, int b) {
  int L = p.Nk;
  if (p.seqlens) {
    L = p.seqlens[b];
    L = L < 0 ? 0 : (L > p.Nk ? p.Nk : L);
  }
  return L;
}

// Keys query row `row` (0 .. Nq-1) may see: the row sits at position
// pos = L - Nq + row (the last Nq positions of the sequence; the one decode
// row at L - 1).  Keys below hc (the valid length, and pos + 1 under the
// causal mask); of those the window keys [lo, hw) (left limit pos - j < w,
// right limit j - pos < wr, each off when 0) and the sink keys [0, sk).
struct RowKeys {
  int lo, hw, sk;
};
__device__ inline RowKeys row_keys(const DecodeParams& p, int L, int row) {
  const int pos = L - p.Nq + row;
  const int hc = max(0, p.causal ? min(L, pos + 1) : L);
  RowKeys r;
  r.hw = p.window_right > 0 ? max(0, min(hc, pos + p.window_right)) : hc;
  r.lo = p.window > 0 ? max(0, pos - p.window + 1) : 0;
  r.sk = min(p.sinks, hc);
  return r;
}
__device__ inline bool key_ok(const RowKeys& r, int j) {
  return j < r.sk || (j >= r.lo && j < r.hw);
}
// First allowed key of a row in [c0, c1) (c1 when none) and the end of its
// allowed keys there (c0 when none).
__device__ inline int split_first(const RowKeys& r, int c0, int c1) {
  int f = c1;
  if (c0 < min(r.sk, c1)) f = c0;
  const int a = max(c0, r.lo), e = min(c1, r.hw);
  if (a < e) f = min(f, a);
  return f;
}
__device__ inline int split_end(const RowKeys& r, int c0, int c1) {
  int e = c0;
  if (c0 < min(r.sk, c1)) e = min(r.sk, c1);
  const int a = max(c0, r.lo), w = min(c1, r.hw);
  if (a < w) e = max(e, w);
  return e;
}

__device__ inline float wave_max(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
// Minimum / maximum over the 16 lanes of each row (lanes 16r .. 16r+15),
// left in every lane of the row: rotations of the row by 8, 4, 2 and 1
// through DPP, with no LDS round trip.
__device__ inline int row_min_i(int x) {
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x122, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x121, 0xF, 0xF, false));
  return x;
}
__device__ inline int row_max_i(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x122, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x121, 0xF, 0xF, false));
  return x;
}

// 16-byte chunk c of tile row r (rows of D * 2 bytes) sits at chunk
// c ^ tile_swz(r): with it the K operand reads (16 rows, one chunk, per 16
// lanes) and the V transposing reads (8 rows x 32 bytes per 32 lanes) touch
// every LDS bank once.
template <int D>
__device__ inline int tile_swz(int r) {
  if constexpr (D == 128)
    return 2 * (r & 7) + ((r >> 3) & 1);
  else
    return 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
}

// a and b start as two copies of x; afterwards {a, b} = {x, x of lane l ^ 16}
// (permlane16) or {x, x of lane l ^ 32} (permlane32) in every lane.  Inline
// assembly with two distinct registers: given the same value twice, the
// builtins were folded to a single result.
__device__ inline void swap16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ inline void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// max / sum over the four lanes n, n + 16, n + 32, n + 48
__device__ inline float quad_max(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = fmaxf(a, b);
  a = x;
  b = x;
  swap32(a, b);
  return fmaxf(a, b);
}
__device__ inline float quad_sum(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = a + b;
  a = x;
  b = x;
  swap32(a, b);
  return a + b;
}

// One tile's matrix operands from LDS: the K rows (ds_read_b128) and the V^T
// blocks (ds_read_b64_tr_b16) of D = 128 or 64, issued together and awaited
// in the same block.  Written as assembly so that the compiler's own wait
// insertion, which cannot tell the stage being read from the stages being
// filled by direct-to-LDS loads at a loop head, adds no wait for those loads:
// the explicit wait on the load counter before each tile orders them.
__device__ inline void lds_operands(bf16x8 (&ka)[4], i16x4 (&va)[8],
                                    const unsigned (&kad)[4],
                                    const unsigned (&vad)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b64_tr_b16 %4, %16\n\t"
      "ds_read_b64_tr_b16 %5, %17\n\t"
      "ds_read_b64_tr_b16 %6, %18\n\t"
      "ds_read_b64_tr_b16 %7, %19\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %21\n\t"
      "ds_read_b64_tr_b16 %10, %22\n\t"
      "ds_read_b64_tr_b16 %11, %23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(ka[0]), "=&v"(ka[1]), "=&v"(ka[2]), "=&v"(ka[3]),
        "=&v"(va[0]), "=&v"(va[1]), "=&v"(va[2]), "=&v"(va[3]),
        "=&v"(va[4]), "=&v"(va[5]), "=&v"(va[6]), "=&v"(va[7])
      : "v"(kad[0]), "v"(kad[1]), "v"(kad[2]), "v"(kad[3]), "v"(vad[0]),
        "v"(vad[1]), "v"(vad[2]), "v"(vad[3]), "v"(vad[4]), "v"(vad[5]),
        "v"(vad[6]), "v"(vad[7])
      : "memory");
}
__device__ inline void lds_operands(bf16x8 (&ka)[2], i16x4 (&va)[4],
                                    const unsigned (&kad)[2],
                                    const unsigned (&vad)[4]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b64_tr_b16 %2, %8\n\t"
      "ds_read_b64_tr_b16 %3, %9\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(ka[0]), "=&v"(ka[1]), "=&v"(va[0]), "=&v"(va[1]),
        "=&v"(va[2]), "=&v"(va[3])
      : "v"(kad[0]), "v"(kad[1]), "v"(vad[0]), "v"(vad[1]), "v"(vad[2]),
        "v"(vad[3])
      : "memory");
}

template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

template <int D>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int TB = kKT * D * 2;    // bytes of one K (or V) tile
  constexpr int TL = TB / 1024;      // wave-wide 16-byte loads per tile
  constexpr int NJ = D / 32;         // k-steps of S^T = K Q^T
  constexpr int NDB = D / 16;        // 16-row blocks of O^T
  constexpr int S = kStages;
  constexpr int ROW = D * 2;         // bytes per tile row
  static_assert(TL * 1024 == TB, "tile loads");
  static_assert(S >= 2 && S <= 6, "stages");
  // one LDS object per stage and operand: the compiler keeps per-object
  // alias scopes, so reads of one stage need not wait for the loads that
  // fill another
#define MIATTN_DSTAGE(X, I) \
  __shared__ __attribute__((aligned(16))) unsigned char X##I[S > I ? TB : 16];
  MIATTN_DSTAGE(Ks, 0) MIATTN_DSTAGE(Ks, 1) MIATTN_DSTAGE(Ks, 2)
  MIATTN_DSTAGE(Ks, 3) MIATTN_DSTAGE(Ks, 4) MIATTN_DSTAGE(Ks, 5)
  MIATTN_DSTAGE(Vs, 0) MIATTN_DSTAGE(Vs, 1) MIATTN_DSTAGE(Vs, 2)
  MIATTN_DSTAGE(Vs, 3) MIATTN_DSTAGE(Vs, 4) MIATTN_DSTAGE(Vs, 5)
#undef MIATTN_DSTAGE
  auto kst = [&](auto st_c) -> unsigned char* {
    constexpr int ST = decltype(st_c)::value;
    if constexpr (ST == 0) return Ks0;
    else if constexpr (ST == 1) return Ks1;
    else if constexpr (ST == 2) return Ks2;
    else if constexpr (ST == 3) return Ks3;
    else if constexpr (ST == 4) return Ks4;
    else return Ks5;
  };
  auto vst = [&](auto st_c) -> unsigned char* {
    constexpr int ST = decltype(st_c)::value;
    if constexpr (ST == 0) return Vs0;
    else if constexpr (ST == 1) return Vs1;
    else if constexpr (ST == 2) return Vs2;
    else if constexpr (ST == 3) return Vs3;
    else if constexpr (ST == 4) return Vs4;
    else return Vs5;
  };

  // grid x = (batch, K/V head, head chunk), fastest; grid y = split.
  // Workgroups are dealt to the XCDs round-robin in launch order, so each
  // XCD sees every split index equally often, whatever the valid lengths.
  const int s = blockIdx.y;
  const int nx = p.Hkv * p.nhc;
  const int b = udiv(blockIdx.x, p.dv_nx);
  const int hk = udiv(blockIdx.x - b * nx, p.dv_nhc);
  const int hc = blockIdx.x - b * nx - hk * p.nhc;
  const int lane = threadIdx.x;
  const int n = lane & 15;   // MFMA column (S^T, O^T), key row (K)
  const int qg = lane >> 4;  // lane group
  // column n of this block: query head hk*G + cl / Nq, row cl % Nq
  const int cl = hc * 16 + n;
  const bool cvalid = cl < p.ncols;
  const int hh = cvalid ? udiv(cl, p.dv_nq) : 0;
  const int row = cvalid ? cl - hh * p.Nq : 0;
  const size_t qrow = ((size_t)(b * p.Hq + hk * p.G + hh)) * p.Nq + row;

  // Q^T operand: column n, features 32j + 8qg .. +7 (zero for padding
  // columns); issued before the valid length is known, the address does not
  // depend on it
  bf16x8 qf[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (cvalid)
      raw = *reinterpret_cast<const u32x4*>(p.q + qrow * D + 32 * j + 8 * qg);
    qf[j] = __builtin_bit_cast(bf16x8, raw);
  }

  const int L = valid_len(p, b);
  RowKeys rk = row_keys(p, L, row);
  if (!cvalid) rk = {0, 0, 0};  // a padding column sees no key
  // this split's keys [c0, c0 + chunk): the block's allowed keys there run
  // from a0 to c1 (the union over its columns)
  const int c0 = s * p.chunk;
  const int cend = c0 + p.chunk;
  // (a lane's keys depend only on its column n, so the four rows of the
  // wave hold the same 16 values and a row's extremum is the wave's)
  const int a0 =
      __builtin_amdgcn_readfirstlane(row_min_i(split_first(rk, c0, cend)));
  const int c1 =
      __builtin_amdgcn_readfirstlane(row_max_i(split_end(rk, c0, cend)));
  if (a0 >= c1) return;  // no allowed key here; the combine skips this split
  const int kt0 = c0 + (a0 - c0) / kKT * kKT;  // first key of the first tile
  const int nt = (c1 - kt0 + kKT - 1) / kKT;   // tiles of this split

  const size_t kv_base = (size_t)(b * p.Hkv + hk) * p.Nk * D;
  const uint16_t* kg = p.k + kv_base;
  const uint16_t* vg = p.v + kv_base;

  // direct-to-LDS placement: load i of a tile fills bytes [i*1024, +1024);
  // lane l writes 16-byte slot i*64 + l = (row r, chunk pc), which holds
  // logical chunk pc ^ tile_swz(r) of key row r.  Every lane loads on every
  // step (the in-order load counter then tells when a stage has landed); a
  // row outside [a0, c1) is clamped to an allowed row, read again from cache,
  // and masked out of the softmax.
  int lrow[TL];
  int lcol[TL];
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    const int slot = i * 64 + lane;
    lrow[i] = slot / CH;
    lcol[i] = ((slot % CH) ^ tile_swz<D>(slot / CH)) * 8;
  }
  auto issue = [&](int t, auto st_c) {
    const int key0 = kt0 + t * kKT;
#pragma unroll
    for (int i = 0; i < TL; ++i) {
      const int key = min(max(key0 + lrow[i], a0), c1 - 1);
      const size_t off = (size_t)key * D + lcol[i];
      __builtin_amdgcn_global_load_lds(
          kg + off, (lds_void*)(kst(st_c) + i * 1024), 16, 0, kNonTemporal);
      __builtin_amdgcn_global_load_lds(
          vg + off, (lds_void*)(vst(st_c) + i * 1024), 16, 0, kNonTemporal);
    }
  };

  // operand read offsets within a stage: K row n, logical chunk 4j + qg
  // (ds_read_b128); V^T block db: lane n of group qg addresses row
  // 4qg + n/4, columns 16db + 4(n%4) .. +3 (ds_read_b64_tr_b16 hands lane n
  // column 16db + n of rows 4qg .. 4qg + 3)
  int koff[NJ], voff[NDB];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    koff[j] = n * ROW + ((4 * j + qg) ^ tile_swz<D>(n)) * 16;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int r = 4 * qg + (n >> 2);
    const int col = 16 * db + 4 * (n & 3);
    voff[db] = r * ROW + ((col >> 3) ^ tile_swz<D>(r)) * 16 + (n & 1) * 8;
  }

  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = {0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY;  // running maximum of head n (log2 units)
  float lsum = 0.f;     // this lane's share of head n's sum

  static_for<0, S - 1>([&](auto r_c) { issue(r_c, r_c); });
  for (int i0 = 0; i0 < nt; i0 += S) {
    static_for<0, S>([&](auto r_c) {
      constexpr int r = decltype(r_c)::value;
      const int t = i0 + r;
      // keep S - 1 tiles in flight: refill the stage read last step
      issue(t + S - 1, ic<(r + S - 1) % S>());
      wait_vm<2 * TL * (S - 1)>();  // tile t has landed
      if (t < nt) {
        // LDS byte addresses of this stage's operands
        const unsigned kb = (unsigned)(uintptr_t)(lds_void*)kst(r_c);
        const unsigned vb = (unsigned)(uintptr_t)(lds_void*)vst(r_c);
        unsigned kad[NJ], vad[NDB];
#pragma unroll
        for (int j = 0; j < NJ; ++j) kad[j] = kb + koff[j];
#pragma unroll
        for (int db = 0; db < NDB; ++db) vad[db] = vb + voff[db];
        bf16x8 ka[NJ];
        i16x4 va[NDB];
        lds_operands(ka, va, kad, vad);
        // S^T = K . Q^T: lane (qg, n) gets keys 4qg + e of head n
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[j], qf[j], sacc, 0,
                                                         0, 0);
        const int key0 = kt0 + t * kKT;
        // no mask when every column allows all keys of the tile (padding
        // columns count as allowing them: their results are never written)
        const bool tile_ok = !cvalid ||
                             (key0 >= rk.lo && key0 + kKT <= rk.hw) ||
                             key0 + kKT <= rk.sk;
        const bool full = __builtin_amdgcn_ballot_w64(!tile_ok) == 0;
        float sc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[e] = sacc[e] * p.c;
          if (!full && !key_ok(rk, key0 + 4 * qg + e)) sc[e] = -INFINITY;
        }
        const float mx =
            quad_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
        // move the running maximum only when a score exceeds it by more
        // than 2^tau (any common shift of a row's scores is exact)
        if (__builtin_amdgcn_ballot_w64(mx > M + kTau)) {
          const float mn = fmaxf(M, mx);
          const float alpha =
              M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mn);
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
          M = mn;
        }
        const float mu = M == -INFINITY ? 0.f : M;
        f32x4 pw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pw[e] = __builtin_amdgcn_exp2f(sc[e] - mu);
          lsum += pw[e];
        }
        const i16x4 pb =
            __builtin_bit_cast(i16x4, __builtin_convertvector(pw, bf16x4));
        // O^T += V^T . P^T
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              va[db], pb, oacc[db], 0, 0, 0);
      }
    });
  }
  // the last loads (clamped rows past the chunk) land before the wave ends
  wait_vm<0>();

  const float lt = quad_sum(lsum);
  if (cvalid) {
    // a column with no allowed key in this split (possible when the block
    // holds several rows) writes o = 0, lse = -inf; the combine reads only
    // the splits that hold keys of its row
    const size_t wrow = qrow * p.nsplit + s;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(p.ws_o + wrow * D + 16 * db + 4 * qg) =
          oacc[db] * inv;
    if (qg == 0)
      p.ws_lse[wrow] =
          lt > 0.f ? (M + log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

// One wavefront per (batch, query head, row); lane l owns features
// l*CPL .. +CPL-1.
template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void decode_combine_kernel(
    DecodeParams p) {
  constexpr int CPL = D / 64;
  const int r = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (r >= p.B * p.Hq * p.Nq) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int b = r / (p.Hq * p.Nq);
  const int row = r - udiv(r, p.dv_nq) * p.Nq;
  const int L = valid_len(p, b);
  const RowKeys rk = row_keys(p, L, row);
  const size_t row0 = (size_t)r * p.nsplit;
  uint16_t* orow = p.o + (size_t)r * D + lane * CPL;
  if (rk.sk == 0 && rk.lo >= rk.hw) {  // no allowed key
#pragma unroll
    for (int e = 0; e < CPL; ++e) orow[e] = 0;
    if (lane == 0 && p.lse) p.lse[r] = -INFINITY;
    return;
  }
  // the splits holding keys of this row (their blocks wrote them)
  const int s0 = rk.sk > 0 ? 0 : udiv(rk.lo, p.dv_chunk);
  const int s1 = udiv(max(rk.hw, rk.sk) + p.chunk - 1, p.dv_chunk);
  auto live = [&](int s) {
    const int c0 = s * p.chunk;
    return split_first(rk, c0, c0 + p.chunk) < c0 + p.chunk;
  };
  float m = -INFINITY;
  for (int s = s0 + lane; s < s1; s += 64)
    if (live(s)) m = fmaxf(m, p.ws_lse[row0 + s]);
  m = wave_max(m);
  float acc[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
  float wsum = 0.f;
#pragma unroll 4
  for (int s = s0; s < s1; ++s) {
    if (!live(s)) continue;  // wave-uniform
    const float w = expf(p.ws_lse[row0 + s] - m);
    wsum += w;
    const float* src = p.ws_o + (row0 + s) * D + lane * CPL;
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[e] = fmaf(w, src[e], acc[e]);
  }
  const float inv = 1.0f / wsum;
#pragma unroll
  for (int e = 0; e < CPL; ++e)
    orow[e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[e] * inv));
  if (lane == 0 && p.lse) p.lse[r] = m + logf(wsum);
}

// Column blocks of one K/V head: its G query heads times Nq rows, 16 per
// wavefront.
long long column_blocks(const Problem& pr) {
  const long long ncols = (long long)(pr.Hq / pr.Hkv) * pr.Nq;
  return (ncols + kCols - 1) / kCols;
}

}  // namespace

// The largest chunk that still gives every decode wavefront slot of the chip
// a split (counting the keys a row may see: the valid length is only known
// on the device, so Nk, or the window plus the sinks plus the rows, bounds
// it), and no smaller than the grid's split limit allows.
int decode_chunk(const Problem& pr) {
  const long long groups = (long long)pr.B * pr.Hkv * column_blocks(pr);
  long long keys = pr.Nk;
  if (pr.window > 0)
    keys = std::min(keys, (long long)pr.window + std::max(pr.sinks, 0) +
                              pr.Nq);
  int chunk = kMaxChunk;
  while (chunk > kMinChunk && groups * ((keys + chunk - 1) / chunk) < kSlots)
    chunk /= 2;
  while ((pr.Nk + (long long)chunk - 1) / chunk > kMaxSplits) chunk *= 2;
  return chunk;
}

bool decode_takes(const Problem& pr) {
  return pr.Nq == 1 ||
         (pr.Nq < pr.Nk && column_blocks(pr) <= kMaxColumnBlocks);
}

size_t decode_workspace_bytes(const Problem& pr) {
  const int chunk = decode_chunk(pr);
  const size_t nsplit = (size_t)((pr.Nk + chunk - 1) / chunk);
  const size_t rows = (size_t)pr.B * pr.Hq * pr.Nq * nsplit;
  return rows * (size_t)pr.d * sizeof(float) + rows * sizeof(float);
}

hipError_t launch_decode_bf16(const void* q, const void* k, const void* v,
                              void* o, float* lse, const Problem& pr, void* ws,
                              hipStream_t stream) {
  DecodeParams p;
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
  p.ncols = p.G * pr.Nq;
  p.nhc = (int)column_blocks(pr);
  p.causal = pr.causal;
  p.window = pr.window;
  p.window_right = pr.window_right;
  p.sinks = pr.sinks;
  p.chunk = decode_chunk(pr);
  p.nsplit = (pr.Nk + p.chunk - 1) / p.chunk;
  p.c = pr.scale * 1.4426950408889634f;
  p.dv_nx = make_udiv(p.Hkv * p.nhc);
  p.dv_nhc = make_udiv(p.nhc);
  p.dv_nq = make_udiv(p.Nq);
  p.dv_chunk = make_udiv(p.chunk);
  const size_t rows = (size_t)pr.B * pr.Hq * pr.Nq * p.nsplit;
  p.ws_o = static_cast<float*>(ws);
  p.ws_lse = p.ws_o + rows * pr.d;
  const int ncomb =
      (int)(((long long)pr.B * pr.Hq * pr.Nq + kCombineWaves - 1) /
            kCombineWaves);
  const dim3 grid(p.B * p.Hkv * p.nhc, p.nsplit);
  if (pr.d == 128) {
    hipLaunchKernelGGL(decode_split_kernel<128>, grid, dim3(64), 0, stream, p);
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(ncomb),
                       dim3(64 * kCombineWaves), 0, stream, p);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<64>, grid, dim3(64), 0, stream, p);
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(ncomb),
                       dim3(64 * kCombineWaves), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace miattn
