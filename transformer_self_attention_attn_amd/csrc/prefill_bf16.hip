// Tiled bf16 prefill attention on gfx950 matrix cores (Nq == Nk).
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
//   workgroup = 4 wavefronts = 128 query rows of one head; wave w owns rows
//   q0 + 32w .. q0 + 32w + 31.  The K/V tile loop walks 64-key tiles that at
//   least one row of the workgroup may see (tiles entirely above the causal
//   diagonal, left of the window or past the valid length are never loaded);
//   a wave skips the arithmetic of tiles that none of its rows may see, and
//   only tiles that are partly allowed pay for per-element masking.
//   Query heads of one K/V head are adjacent in the launch order and the
//   block index is remapped so that each XCD (own L2) works on a contiguous
//   range of (batch, K/V head) groups; causal blocks run heaviest first.
//
// Per tile, per wave (the transposed formulation keeps each query's softmax
// statistics inside one lane pair):
//   S^T[key][query] = K_tile . Q^T     v_mfma_f32_32x32x16_bf16, A = K rows
//                                      from LDS, B = Q^T held in registers
//   online softmax in base 2 (scale * log2 e folded into one FMA); the
//   running maximum is only moved (and O rescaled) when some row's new
//   maximum exceeds it by more than 2^8, which is exact arithmetic: the
//   stored maximum is any common shift of the row's scores
//   O^T[d][query] += V^T . P^T         A = V^T from LDS (V is transposed on
//                                      its way into LDS), B = P^T (bf16) taken
//                                      straight from the S^T accumulator
// K/V tiles are double-buffered in LDS and the next tile's global loads are
// issued before the current tile's matrix work.
#include "kernels.h"

#include <cmath>

namespace miattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;             // query rows per wavefront
constexpr int kQB = kQW * kWaves;   // query rows per workgroup
constexpr int kKT = 64;             // keys per tile
constexpr float kTau = 8.0f;        // lazy-rescale threshold, log2 units
constexpr int kXcds = 8;            // MI355X: 8 accelerator complex dies

template <int D>
struct Cfg {
  static constexpr int KSTR = D + 8;      // K tile row stride in LDS (elements)
  static constexpr int VSTR = kKT + 8;    // V^T tile row stride (elements)
  static constexpr int KBUF = kKT * KSTR;
  static constexpr int VBUF = D * VSTR;
  static constexpr int KCH = kKT * D / 8;             // 16-byte chunks per tile
  static constexpr int KCH_T = KCH / kThreads;        // per thread
  static constexpr int VUNITS = (kKT / 4) * (D / 8);  // 4 keys x 8 columns
  static constexpr int VU_T = (VUNITS + kThreads - 1) / kThreads;
  static constexpr int KS = D / 16;  // k-steps of the S^T product
  static constexpr int DB = D / 32;  // 32-row blocks of O^T
  static_assert(KCH % kThreads == 0, "K tile split");
};

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* seqlens;
  int B, Hq, Hkv, N, G, nqb, causal, window, total;
  float c;         // |scale| * log2(e)
  unsigned qsign;  // 0x80008000 when scale < 0: Q is negated on load
};

__device__ inline unsigned perm(unsigned hi_src, unsigned lo_src,
                                unsigned sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// Row of the K tile in LDS that feeds MFMA row rho of key block mb.  Keys are
// stored permuted so that, in the 32x32 accumulator layout, lane group g of
// the S^T result holds the 16 consecutive keys g*16 .. g*16+15 of the block.
__device__ inline int k_lds_row(int key_in_tile) {
  const int mb = key_in_tile >> 5;
  const int kk = key_in_tile & 31;
  const int rho = ((kk >> 2) & 3) * 8 + ((kk >> 4) & 1) * 4 + (kk & 3);
  return mb * 32 + rho;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][C::VBUF];

  // ---- block -> (batch, head, query block) --------------------------------
  const int n = p.total;
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int slot = bid / kXcds;
  const int per = n / kXcds;
  const int rem = n % kXcds;
  const int lid = xcd * per + min(xcd, rem) + slot;

  const int per_grp = p.G * p.nqb;
  const int grp = lid / per_grp;
  const int r0 = lid - grp * per_grp;
  const int qrank = r0 / p.G;
  const int hh = r0 - qrank * p.G;
  const int qb = p.causal ? (p.nqb - 1 - qrank) : qrank;
  const int b = grp / p.Hkv;
  const int hk = grp - b * p.Hkv;
  const int h = hk * p.G + hh;

  int L = p.N;
  if (p.seqlens) {
    L = p.seqlens[b];
    L = L < 0 ? 0 : (L > p.N ? p.N : L);
  }
  // Nq == Nk: the first L rows are live and row i sits at position i.

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int g = lane >> 5;
  const int q0 = qb * kQB;
  const int qw0 = q0 + wave * kQW;
  const int qi = qw0 + ql;

  const size_t qo_base = (size_t)(b * p.Hq + h) * p.N * D;
  const size_t kv_base = (size_t)(b * p.Hkv + hk) * p.N * D;
  const uint16_t* kg = p.k + kv_base;
  const uint16_t* vg = p.v + kv_base;

  // ---- key ranges ---------------------------------------------------------
  const bool qlive = qi < L;
  const int hi = qlive ? (p.causal ? min(L, qi + 1) : L) : 0;  // exclusive
  const int lo = (qlive && p.window > 0) ? max(0, qi - p.window + 1) : 0;

  const int rows_end = min(q0 + kQB, L);
  int t0 = 0, t1 = 0;
  if (rows_end > q0) {
    const int kv_hi = p.causal ? min(L, rows_end) : L;
    const int kv_lo = p.window > 0 ? max(0, q0 - p.window + 1) : 0;
    t0 = kv_lo / kKT;
    t1 = (kv_hi + kKT - 1) / kKT;
  }
  const int wend = min(qw0 + kQW, L);
  const bool wlive = wend > qw0;
  const int w_hi_max = p.causal ? min(L, wend) : L;
  const int w_hi_min = p.causal ? min(L, qw0 + 1) : L;
  const int w_lo_min = p.window > 0 ? max(0, qw0 - p.window + 1) : 0;
  const int w_lo_max = p.window > 0 ? max(0, wend - 1 - p.window + 1) : 0;

  // ---- Q^T fragments (B operand), kept in registers -----------------------
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qlive) {
      raw = *reinterpret_cast<const u32x4*>(p.q + qo_base + (size_t)qi * D +
                                            16 * ks + 8 * g);
      raw ^= p.qsign;
    }
    qf[ks] = __builtin_bit_cast(bf16x8, raw);
  }

  // ---- tile staging -------------------------------------------------------
  u32x4 kr[C::KCH_T];
  u32x4 vr[4 * C::VU_T];
  auto gload = [&](int t) {
    const int j0 = t * kKT;
#pragma unroll
    for (int i = 0; i < C::KCH_T; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch / (D / 8);
      const int col = ch % (D / 8);
      const int key = j0 + row;
      kr[i] = (key < L) ? *reinterpret_cast<const u32x4*>(
                              kg + (size_t)key * D + col * 8)
                        : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < C::VU_T; ++i) {
      const int u = tid + kThreads * i;
      const int kq = u % (kKT / 4);
      const int dc = u / (kKT / 4);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = j0 + 4 * kq + rr;
        vr[4 * i + rr] = (u < C::VUNITS && key < L)
                             ? *reinterpret_cast<const u32x4*>(
                                   vg + (size_t)key * D + dc * 8)
                             : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KCH_T; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch / (D / 8);
      const int col = ch % (D / 8);
      *reinterpret_cast<u32x4*>(&Ks[buf][k_lds_row(row) * C::KSTR + col * 8]) =
          kr[i];
    }
#pragma unroll
    for (int i = 0; i < C::VU_T; ++i) {
      const int u = tid + kThreads * i;
      if (u < C::VUNITS) {
        const int kq = u % (kKT / 4);
        const int dc = u / (kKT / 4);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const unsigned a0 = vr[4 * i + 0][cc], a1 = vr[4 * i + 1][cc];
          const unsigned a2 = vr[4 * i + 2][cc], a3 = vr[4 * i + 3][cc];
          // column d = dc*8 + 2cc takes the low halves, d + 1 the high halves
          const u32x2 lo2 = {perm(a1, a0, 0x05040100u),
                             perm(a3, a2, 0x05040100u)};
          const u32x2 hi2 = {perm(a1, a0, 0x07060302u),
                             perm(a3, a2, 0x07060302u)};
          const int d0 = dc * 8 + 2 * cc;
          *reinterpret_cast<u32x2*>(&Vs[buf][d0 * C::VSTR + 4 * kq]) = lo2;
          *reinterpret_cast<u32x2*>(&Vs[buf][(d0 + 1) * C::VSTR + 4 * kq]) =
              hi2;
        }
      }
    }
  };

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float M = -INFINITY;  // running maximum of s * c (log2 units)
  float l = 0.f;        // this lane's half of the running sum

  if (t1 > t0) {
    gload(t0);
    lstore(0);
  }
  __syncthreads();

  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    if (t + 1 < t1) gload(t + 1);
    const int j0 = t * kKT;
    const bool skip = !wlive || j0 >= w_hi_max || j0 + kKT <= w_lo_min;
    if (!skip) {
      const bool full = j0 >= w_lo_max && j0 + kKT <= w_hi_min;
      f32x16 sacc[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[mb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              &Ks[buf][(mb * 32 + ql) * C::KSTR + 16 * ks + 8 * g]);
          sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks],
                                                             sacc[mb], 0, 0, 0);
        }
      }
      // lane holds keys j0 + mb*32 + g*16 + r (r = 0..15) of query qi
      if (!full) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + mb * 32 + g * 16 + r;
            if (j < lo || j >= hi) sacc[mb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
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
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s = sacc[mb][r];
          float e = __builtin_amdgcn_exp2f(fmaf(s, p.c, -mu));
          if (!full) e = (s == -INFINITY) ? 0.f : e;
          sacc[mb][r] = e;
          l += e;
        }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          f32x8 pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = sacc[mb][8 * m + e];
          const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                &Vs[buf][(db * 32 + ql) * C::VSTR + mb * 32 + 16 * g + 8 * m]);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db],
                                                               0, 0, 0);
          }
        }
    }
    if (t + 1 < t1) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -----------------------------------------------------------
  const float lt = l + __shfl_xor(l, 32);
  if (qi < p.N) {
    const bool any = qlive && lt > 0.f;
    const float inv = any ? 1.f / lt : 0.f;
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
      p.lse[(size_t)(b * p.Hq + h) * p.N + qi] =
          any ? (M + log2f(lt)) * 0.69314718055994531f : -INFINITY;
    }
  }
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
  p.N = pr.Nq;
  p.G = pr.Hq / pr.Hkv;
  p.nqb = (pr.Nq + kQB - 1) / kQB;
  p.causal = pr.causal;
  p.window = pr.window;
  p.total = pr.B * pr.Hq * p.nqb;
  p.c = fabsf(pr.scale) * 1.4426950408889634f;
  p.qsign = (pr.scale < 0.f) ? 0x80008000u : 0u;
  if (pr.d == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, dim3(p.total), dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL(prefill_kernel<64>, dim3(p.total), dim3(kThreads), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace miattn
