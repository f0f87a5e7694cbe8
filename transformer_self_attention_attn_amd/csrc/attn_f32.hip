// fp32 attention: one wavefront per output row, fp32 arithmetic end to end.
//
// Computes, for query row i of head h (K/V head h / G):
//   s_j = scale * q_i . k_j over allowed keys j,
//   o_i = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),  lse_i = m + ln sum
// (score and softmax as in the SpAtten review page, Background - Attention
// Mechanism; masks as in the self-attention explainer page, Padding and
// Look-Ahead Masking, and the tutorial page's Local Window Attention).
// Keys are visited in tiles of 64 (one key per lane) with a running maximum
// and sum, so the result is the exact softmax up to fp32 rounding.
#include "kernels.h"

#include <cmath>

namespace miattn {
namespace {

constexpr int kRowsPerBlock = 4;  // one row per wavefront

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int* seqlens;
  int B, Hq, Hkv, Nq, Nk, G, causal, window, window_right, sinks;
  float scale;
  long long rows;
};

__device__ inline float wave_max(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ inline float wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(F32Params p) {
  constexpr int C = D / 64;  // output columns per lane
  __shared__ float qs[kRowsPerBlock][D];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + wave;
  if (row >= p.rows) return;  // whole wavefront leaves together

  const int i = (int)(row % p.Nq);
  const long long bh = row / p.Nq;
  const int h = (int)(bh % p.Hq);
  const int b = (int)(bh / p.Hq);
  const int hk = h / p.G;

  int L = p.Nk;
  if (p.seqlens) {
    L = p.seqlens[b];
    L = L < 0 ? 0 : (L > p.Nk ? p.Nk : L);
  }
  const int live_rows = (p.Nq == p.Nk) ? L : p.Nq;
  const int pos = i + (L - live_rows);
  const bool live = i < live_rows;
  // allowed keys: [0, sa) (sink keys) and [lo, hi) (the window), both cut
  // to the causal and padding limit hc
  const int hc = live ? (p.causal ? min(L, pos + 1) : L) : 0;  // exclusive
  const int lo = (live && p.window > 0) ? max(0, pos - p.window + 1) : 0;
  const int hi = p.window_right > 0 ? min(hc, pos + p.window_right) : hc;
  const int sa = min(p.sinks, hc);

  const float* qrow = p.q + (size_t)row * D;
  const float* kb = p.k + (size_t)(b * p.Hkv + hk) * p.Nk * D;
  const float* vb = p.v + (size_t)(b * p.Hkv + hk) * p.Nk * D;
  if (live) {
    for (int c = 0; c < C; ++c) qs[wave][lane + 64 * c] = qrow[lane + 64 * c];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

  float acc[C];
  for (int c = 0; c < C; ++c) acc[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  // online softmax over the keys of [jlo, jhi)
  auto sweep = [&](int jlo, int jhi) {
    for (int j0 = jlo; j0 < jhi; j0 += 64) {
      const int j = j0 + lane;
      const bool ok = j < jhi;
      const int nj = min(64, jhi - j0);
      // the tile's V rows, all loads issued ahead of the scores, so their
      // latency overlaps the K loads' instead of adding to it (rows past nj
      // repeat row j0 and are weighted by 0)
      float vv[64][C];
#pragma unroll
      for (int u = 0; u < 64; ++u) {
        const float* vr = vb + (size_t)(j0 + (u < nj ? u : 0)) * D;
#pragma unroll
        for (int c = 0; c < C; ++c) vv[u][c] = vr[lane + 64 * c];
      }
      float s = -INFINITY;
      if (ok) {
        const float4* kr = reinterpret_cast<const float4*>(kb + (size_t)j * D);
        float dot = 0.f;
        for (int c4 = 0; c4 < D / 4; ++c4) {
          const float4 kk = kr[c4];
          dot = fmaf(qs[wave][4 * c4 + 0], kk.x, dot);
          dot = fmaf(qs[wave][4 * c4 + 1], kk.y, dot);
          dot = fmaf(qs[wave][4 * c4 + 2], kk.z, dot);
          dot = fmaf(qs[wave][4 * c4 + 3], kk.w, dot);
        }
        s = dot * p.scale;
      }
      const float mn = fmaxf(m, wave_max(s));  // finite: lane 0 is allowed
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
      const float pj = ok ? expf(s - mn) : 0.f;
      l = l * alpha + wave_sum(pj);
      for (int c = 0; c < C; ++c) acc[c] *= alpha;
#pragma unroll
      for (int u = 0; u < 64; ++u) {
        const float w = __shfl(pj, u);  // 0 past nj: pj = 0 there
#pragma unroll
        for (int c = 0; c < C; ++c) acc[c] = fmaf(w, vv[u][c], acc[c]);
      }
      m = mn;
    }
  };
  sweep(0, sa);
  sweep(max(lo, sa), hi);
  float* orow = p.o + (size_t)row * D;
  const bool any = l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  for (int c = 0; c < C; ++c) orow[lane + 64 * c] = any ? acc[c] * inv : 0.f;
  if (p.lse && lane == 0) p.lse[row] = any ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v,
                           float* o, float* lse, const Problem& pr,
                           hipStream_t stream) {
  F32Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
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
  p.scale = pr.scale;
  p.rows = (long long)pr.B * pr.Hq * pr.Nq;
  const unsigned blocks =
      (unsigned)((p.rows + kRowsPerBlock - 1) / kRowsPerBlock);
  if (pr.d == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(blocks), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(blocks), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace miattn
