// One-token decode attention (Nq == 1), bf16 K/V cache, split over keys.
//
// The generation step processes a single new token whose K and V have been
// appended to the cache (SpAtten review page, Background - Attention-Based NLP
// Models); the page notes this stage is memory-bound.  The query is the last
// token of its sequence: it may see keys j < L_b (and, with a window w, only
// j >= L_b - w).
//
// Pass 1 (decode_split_kernel): grid = splits x (K/V head, head chunk) x batch.
//   A workgroup owns a chunk of kChunk keys of one (batch, K/V head) and the
//   GB query heads of that group that share it, so each K and V byte is read
//   from HBM exactly once for all of them.
//     K sweep: s_hj = scale * q_h . k_j for the chunk (dot products of bf16
//              pairs in fp32, reduced across the lanes that share a key row
//              with DPP), kept in LDS in log2 units;
//     softmax: per head, m_h = max_j s_hj and l_h = sum_j 2^(s_hj - m_h) over
//              the chunk (workgroup reductions);
//     V sweep: o_h = sum_j 2^(s_hj - m_h) v_j / l_h.
//   It writes the chunk's partial result o_s (fp32) and lse_s = (m + log2 l)
//   ln 2 to the workspace.  Chunks that hold no allowed key exit at once.
// Pass 2 (decode_combine_kernel): grid = query heads x batch.
//   lse = log sum_s exp(lse_s) (max-shifted) and o = sum_s exp(lse_s - lse) o_s,
//   the softmax definition applied to a partition of the keys; written as bf16
//   o and fp32 lse.
#include "kernels.h"

#include <cmath>

namespace miattn {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kChunk = 512;  // keys per split
constexpr int kUnroll = 4;   // key rows in flight per lane
constexpr int kMaxGB = 8;    // query heads per workgroup

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* seqlens;
  float* ws_o;    // [B, Hq, nsplit, D]
  float* ws_lse;  // [B, Hq, nsplit]
  int B, Hq, Hkv, Nk, G, GB, nhc, window, nsplit;
  float c;  // scale * log2(e)
};

__device__ inline void key_range(const DecodeParams& p, int b, int& lo,
                                 int& L) {
  L = p.Nk;
  if (p.seqlens) {
    L = p.seqlens[b];
    L = L < 0 ? 0 : (L > p.Nk ? p.Nk : L);
  }
  // the query sits at position L - 1: keys j <= L - 1 (causal or not, no key
  // at or past L is valid); a window keeps L - 1 - j < w, i.e. j >= L - w
  lo = p.window > 0 ? max(0, L - p.window) : 0;
}

template <int W>
__device__ inline float group_sum(float x) {
  // sum over aligned groups of W lanes (W = 8 or 16) with DPP row permutes
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                     __builtin_bit_cast(int, x), 0xB1, 0xF,
                                     0xF, true));  // quad_perm [1,0,3,2]
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                     __builtin_bit_cast(int, x), 0x4E, 0xF,
                                     0xF, true));  // quad_perm [2,3,0,1]
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                     __builtin_bit_cast(int, x), 0x141, 0xF,
                                     0xF, true));  // row_half_mirror
  if (W == 16)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                       __builtin_bit_cast(int, x), 0x140, 0xF,
                                       0xF, true));  // row_mirror
  return x;
}

__device__ inline float wave_max(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ inline float wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ inline float bf16_lo(unsigned w) {
  return __builtin_bit_cast(float, w << 16);
}
__device__ inline float bf16_hi(unsigned w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

template <int D, int GB>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    DecodeParams p) {
  constexpr int LPK = D / 8;             // lanes per key row (16 B each)
  constexpr int KPI = kThreads / LPK;    // key rows per workgroup step
  constexpr int STEPS = kChunk / KPI;
  static_assert(STEPS % kUnroll == 0, "chunk split");
  __shared__ float sc[kChunk * GB];           // scores, then weights
  __shared__ float red[kThreads / 64][GB];    // cross-wave reductions
  __shared__ float ored[kThreads / 64][GB * D];

  const int s = blockIdx.x;
  const int hk = blockIdx.y / p.nhc;
  const int hc = blockIdx.y - hk * p.nhc;
  const int b = blockIdx.z;
  int lo, L;
  key_range(p, b, lo, L);
  const int c0 = s * kChunk;
  const int c1 = min(c0 + kChunk, L);
  const int a0 = max(c0, lo);
  if (a0 >= c1) return;  // no allowed key here; the combine skips this split

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int dch = tid % LPK;  // 8-column chunk of the row this lane reads
  const int krow = tid / LPK;
  const int h0 = hk * p.G + hc * GB;
  const int nh = min(GB, p.G - hc * GB);

  // query fragments: 8 columns of each head, as bf16 pairs
  unsigned qw[GB][4];
#pragma unroll
  for (int gi = 0; gi < GB; ++gi) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (gi < nh)
      raw = *reinterpret_cast<const u32x4*>(
          p.q + (size_t)(b * p.Hq + h0 + gi) * D + dch * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) qw[gi][e] = raw[e];
  }

  const size_t kv_base = (size_t)(b * p.Hkv + hk) * p.Nk * D;
  const uint16_t* kg = p.k + kv_base + dch * 8;
  const uint16_t* vg = p.v + kv_base + dch * 8;

  // ---- K sweep: scores --------------------------------------------------
  for (int it = 0; it < STEPS; it += kUnroll) {
    u32x4 kk[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = c0 + (it + u) * KPI + krow;
      kk[u] = (key >= a0 && key < c1)
                  ? *reinterpret_cast<const u32x4*>(kg + (size_t)key * D)
                  : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = c0 + (it + u) * KPI + krow;
      const bool ok = key >= a0 && key < c1;
#pragma unroll
      for (int gi = 0; gi < GB; ++gi) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // copy the vector element out first: bit-casting the element
          // expression itself would read element 0
          const unsigned kw = kk[u][e];
          const unsigned qv = qw[gi][e];
          acc = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2, kw), __builtin_bit_cast(bf16x2, qv),
              acc, false);
        }
        acc = group_sum<LPK>(acc);
        if (dch == 0)
          sc[(key - c0) * GB + gi] = ok ? acc * p.c : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- chunk softmax statistics per head -------------------------------
  float mh[GB], lh[GB];
#pragma unroll
  for (int gi = 0; gi < GB; ++gi) {
    float m = -INFINITY;
    for (int j = tid; j < kChunk; j += kThreads) m = fmaxf(m, sc[j * GB + gi]);
    m = wave_max(m);
    if (lane == 0) red[wave][gi] = m;
  }
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < GB; ++gi) {
    float m = red[0][gi];
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w][gi]);
    mh[gi] = m;  // finite: the chunk holds at least one allowed key
  }
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < GB; ++gi) {
    float sum = 0.f;
    for (int j = tid; j < kChunk; j += kThreads) {
      const float e = __builtin_amdgcn_exp2f(sc[j * GB + gi] - mh[gi]);
      sc[j * GB + gi] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) red[wave][gi] = sum;
  }
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < GB; ++gi) {
    float sum = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) sum += red[w][gi];
    lh[gi] = sum;
  }

  // ---- V sweep: weighted sum -------------------------------------------
  float o[GB][8];
#pragma unroll
  for (int gi = 0; gi < GB; ++gi)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[gi][e] = 0.f;
  for (int it = 0; it < STEPS; it += kUnroll) {
    u32x4 vv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = c0 + (it + u) * KPI + krow;
      vv[u] = (key >= a0 && key < c1)
                  ? *reinterpret_cast<const u32x4*>(vg + (size_t)key * D)
                  : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int jl = (it + u) * KPI + krow;  // key - c0
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_lo(vv[u][e]);
        x[2 * e + 1] = bf16_hi(vv[u][e]);
      }
#pragma unroll
      for (int gi = 0; gi < GB; ++gi) {
        const float w = sc[jl * GB + gi];  // 0 for keys that are not allowed
#pragma unroll
        for (int e = 0; e < 8; ++e) o[gi][e] = fmaf(w, x[e], o[gi][e]);
      }
    }
  }
  // lanes with the same column chunk hold different keys: add them up
#pragma unroll
  for (int gi = 0; gi < GB; ++gi)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[gi][e];
      for (int m = LPK; m < 64; m <<= 1) x += __shfl_xor(x, m);
      o[gi][e] = x;
    }
  if (lane < LPK) {
#pragma unroll
    for (int gi = 0; gi < GB; ++gi)
#pragma unroll
      for (int e = 0; e < 8; ++e) ored[wave][gi * D + dch * 8 + e] = o[gi][e];
  }
  __syncthreads();
  for (int t = tid; t < nh * D; t += kThreads) {
    const int gi = t / D;
    const int d = t - gi * D;
    float x = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) x += ored[w][t];
    float lsum = 0.f, mval = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < GB; ++g2)
      if (g2 == gi) {
        lsum = lh[g2];
        mval = mh[g2];
      }
    const size_t row = (size_t)(b * p.Hq + h0 + gi) * p.nsplit + s;
    p.ws_o[row * D + d] = x / lsum;
    if (d == 0)
      p.ws_lse[row] = (mval + log2f(lsum)) * 0.69314718055994531f;
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeParams p) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  int lo, L;
  key_range(p, b, lo, L);
  const size_t row0 = (size_t)(b * p.Hq + h) * p.nsplit;
  uint16_t* orow = p.o + (size_t)(b * p.Hq + h) * D;
  if (L <= lo) {  // no allowed key
    orow[d] = 0;
    if (d == 0 && p.lse) p.lse[b * p.Hq + h] = -INFINITY;
    return;
  }
  const int s0 = lo / kChunk;
  const int s1 = (L + kChunk - 1) / kChunk;
  float m = -INFINITY;
  for (int s = s0; s < s1; ++s) m = fmaxf(m, p.ws_lse[row0 + s]);
  float wsum = 0.f, acc = 0.f;
  for (int s = s0; s < s1; ++s) {
    const float w = expf(p.ws_lse[row0 + s] - m);
    wsum += w;
    acc = fmaf(w, p.ws_o[(row0 + s) * D + d], acc);
  }
  const __bf16 ob = (__bf16)(acc / wsum);
  orow[d] = __builtin_bit_cast(uint16_t, ob);
  if (d == 0 && p.lse) p.lse[b * p.Hq + h] = m + logf(wsum);
}

int heads_per_block(int G) {
  if (G <= kMaxGB) return G;
  for (int gb = kMaxGB; gb > 1; --gb)
    if (G % gb == 0) return gb;
  return 1;
}

template <int D, int GB>
void launch_split(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((decode_split_kernel<D, GB>),
                     dim3(p.nsplit, p.Hkv * p.nhc, p.B), dim3(kThreads), 0, st,
                     p);
}

template <int D>
void launch_split_d(const DecodeParams& p, hipStream_t st) {
  switch (p.GB) {
    case 1: launch_split<D, 1>(p, st); break;
    case 2: launch_split<D, 2>(p, st); break;
    case 3: launch_split<D, 3>(p, st); break;
    case 4: launch_split<D, 4>(p, st); break;
    case 5: launch_split<D, 5>(p, st); break;
    case 6: launch_split<D, 6>(p, st); break;
    case 7: launch_split<D, 7>(p, st); break;
    default: launch_split<D, 8>(p, st); break;
  }
}

}  // namespace

size_t decode_workspace_bytes(const Problem& pr) {
  const size_t nsplit = (size_t)((pr.Nk + kChunk - 1) / kChunk);
  const size_t rows = (size_t)pr.B * pr.Hq * nsplit;
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
  p.Nk = pr.Nk;
  p.G = pr.Hq / pr.Hkv;
  p.GB = heads_per_block(p.G);
  p.nhc = (p.G + p.GB - 1) / p.GB;
  p.window = pr.window;
  p.nsplit = (pr.Nk + kChunk - 1) / kChunk;
  p.c = pr.scale * 1.4426950408889634f;
  const size_t rows = (size_t)pr.B * pr.Hq * p.nsplit;
  p.ws_o = static_cast<float*>(ws);
  p.ws_lse = p.ws_o + rows * pr.d;
  if (pr.d == 128) {
    launch_split_d<128>(p, stream);
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(pr.Hq, pr.B),
                       dim3(128), 0, stream, p);
  } else {
    launch_split_d<64>(p, stream);
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(pr.Hq, pr.B), dim3(64),
                       0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace miattn
