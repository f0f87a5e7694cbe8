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
//   from HBM exactly once for all of them.  The chunk is one pass over its
//   key rows: every group of D/8 lanes takes every (kThreads*8/D)-th row,
//   loads its K and V together (16 B per lane each, non-temporal: the cache
//   is streamed once) and keeps, per head, an online softmax of its own rows:
//     s = scale * q . k       (bf16 pair dot products in fp32, summed across
//                              the group's lanes with DPP), in log2 units;
//     m = running maximum, moved (and l, o rescaled) only when a score
//         exceeds it by more than 2^8;
//     l += 2^(s - m);  o += 2^(s - m) v.
//   A register ring keeps the next kRing-1 batches of rows in flight, and
//   nothing waits on other lanes until the chunk ends.  Then the groups are
//   merged (shifts to a common maximum) across lanes and, through LDS,
//   across the wavefronts.  The workgroup writes the chunk's partial result
//   o_s = o / l (fp32) and lse_s = (m + log2 l) ln 2 to the workspace.
//   Chunks that hold no allowed key exit at once.
// Pass 2 (decode_combine_kernel): one wavefront per (batch, query head).
//   lse = log sum_s exp(lse_s) (max-shifted) and o = sum_s exp(lse_s - lse) o_s,
//   the softmax definition applied to a partition of the keys; written as bf16
//   o and fp32 lse.
#include "kernels.h"

#include <cmath>

namespace miattn {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#ifndef MIATTN_DECODE_EAGER
#define MIATTN_DECODE_EAGER 0
#endif
#ifndef MIATTN_DECODE_RING
#define MIATTN_DECODE_RING 4
#endif

constexpr int kThreads = 256;
#ifndef MIATTN_DECODE_CHUNK
#define MIATTN_DECODE_CHUNK 512
#endif
constexpr int kChunk = MIATTN_DECODE_CHUNK;  // keys per split
constexpr int kRing = MIATTN_DECODE_RING;  // key-row batches per lane in flight + 1
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units
constexpr int kMaxGB = 8;    // query heads per workgroup
constexpr int kCombineWaves = 4;  // (batch, head) rows per combine workgroup

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* seqlens;
  float* ws_o;    // [B, Hq, nsplit, D]
  float* ws_lse;  // [B, Hq, nsplit]
  int B, Hq, Hkv, Nk, G, GB, nhc, window, sinks, nsplit;
  float c;  // scale * log2(e)
};

__device__ inline void key_range(const DecodeParams& p, int b, int& lo,
                                 int& L, int& sk) {
  L = p.Nk;
  if (p.seqlens) {
    L = p.seqlens[b];
    L = L < 0 ? 0 : (L > p.Nk ? p.Nk : L);
  }
  // the query sits at position L - 1: keys j <= L - 1 (causal or not, no key
  // at or past L is valid); a window keeps L - 1 - j < w, i.e. j >= L - w
  // (a right limit never removes a key here); sink keys j < sinks stay
  lo = p.window > 0 ? max(0, L - p.window) : 0;
  sk = min(p.sinks, L);
}

// Lowest allowed key of split s ([c0, c1) = its keys before the window and
// sink rules): the split holds sink keys [c0, min(c1, sk)) and window keys
// [max(c0, lo), c1); c1 (no allowed key) when both are empty.
__device__ inline int split_first_key(int c0, int c1, int lo, int sk) {
  if (c0 < sk && c0 < c1) return c0;
  const int a = max(c0, lo);
  return a < c1 ? a : c1;
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

// K and V rows are read once per call: streaming (non-temporal) loads keep
// them from displacing reusable lines in the caches.
__device__ inline u32x4 load_stream(const uint16_t* ptr) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
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
  constexpr int LPK = D / 8;           // lanes per key row (16 B each)
  constexpr int GPW = 64 / LPK;        // row groups per wavefront
  constexpr int NWV = kThreads / 64;   // wavefronts per workgroup
  constexpr int RPB = kThreads / LPK;  // key rows per batch (one per group)
  constexpr int R = kRing;             // batches held in registers
  __shared__ float red_o[NWV][GB * D];
  __shared__ float red_ml[NWV][2 * GB];

  // grid x = (batch, K/V head, head chunk), fastest; grid y = split.
  // Workgroups are dealt to the XCDs round-robin in launch order, so each
  // XCD sees every split index equally often, whatever the valid lengths.
  const int s = blockIdx.y;
  const int nx = p.Hkv * p.nhc;
  const int b = blockIdx.x / nx;
  const int hk = (blockIdx.x - b * nx) / p.nhc;
  const int hc = blockIdx.x - b * nx - hk * p.nhc;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int dch = tid % LPK;  // 8-column chunk of the row this lane reads
  const int grp = tid / LPK;  // row group: rows c0 + i * RPB + grp
  const int h0 = hk * p.G + hc * GB;
  const int nh = min(GB, p.G - hc * GB);

  // query fragments (8 columns of each head as bf16 pairs); issued before
  // the valid length is known, the address does not depend on it
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

  int lo, L, sk;
  key_range(p, b, lo, L, sk);
  const int c0 = s * kChunk;
  const int c1 = min(c0 + kChunk, L);
  const int a0 = split_first_key(c0, c1, lo, sk);
  if (a0 >= c1) return;  // no allowed key here; the combine skips this split
  const int first = (a0 - c0) / RPB;
  const int nb = (c1 - c0 + RPB - 1) / RPB;  // batches first .. nb-1

  const size_t kv_base = (size_t)(b * p.Hkv + hk) * p.Nk * D;
  const uint16_t* kg = p.k + kv_base + dch * 8;
  const uint16_t* vg = p.v + kv_base + dch * 8;

  // ring of R batches: batch i sits in slot (i - first) % R.  Every lane
  // loads on every step (no branch around the loads, so the hardware's
  // in-order load counter tells exactly when a slot has arrived); a row
  // outside [a0, c1) is clamped to an allowed row, read again from cache,
  // and masked out of the softmax.
  u32x4 kr[R], vr[R];
  auto issue = [&](int i, u32x4& kd, u32x4& vd) {
    const int key = min(max(c0 + i * RPB + grp, a0), c1 - 1);
    kd = load_stream(kg + (size_t)key * D);
    vd = load_stream(vg + (size_t)key * D);
  };
#pragma unroll
  for (int r = 0; r < R - 1; ++r) issue(first + r, kr[r], vr[r]);

  // per row group and head: running max m (log2 units), sum l, output o
  float m[GB], l[GB], o[GB][8];
#pragma unroll
  for (int gi = 0; gi < GB; ++gi) {
    m[gi] = -INFINITY;
    l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[gi][e] = 0.f;
  }

  // whole rounds of R steps; steps past the last batch are fully masked
  for (int i0 = first; i0 < nb; i0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = i0 + r;
      {
        // keep R - 1 batches in flight: refill the slot freed last step
        issue(i + R - 1, kr[(r + R - 1) % R], vr[(r + R - 1) % R]);
        const int key = c0 + i * RPB + grp;
        const bool ok = key >= a0 && key < c1 && (key >= lo || key < sk);
        float sc[GB];
#pragma unroll
        for (int gi = 0; gi < GB; ++gi) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned kw = kr[r][e];
            const unsigned qv = qw[gi][e];
            acc = __builtin_amdgcn_fdot2_f32_bf16(
                __builtin_bit_cast(bf16x2, kw), __builtin_bit_cast(bf16x2, qv),
                acc, false);
          }
          acc = group_sum<LPK>(acc);
          sc[gi] = ok ? acc * p.c : -INFINITY;
        }
        // move the running maximum only when a score exceeds it by more
        // than 2^tau (any common shift of a row's scores is exact)
#if MIATTN_DECODE_EAGER
        {
#else
        bool grow = false;
#pragma unroll
        for (int gi = 0; gi < GB; ++gi) grow |= sc[gi] > m[gi] + kTau;
        if (__builtin_amdgcn_ballot_w64(grow)) {
#endif
#pragma unroll
          for (int gi = 0; gi < GB; ++gi) {
            const float mn = fmaxf(m[gi], sc[gi]);
            const float a =
                mn == m[gi] ? 1.0f : __builtin_amdgcn_exp2f(m[gi] - mn);
            m[gi] = mn;
            l[gi] *= a;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[gi][e] *= a;
          }
        }
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned vw = vr[r][e];
          x[2 * e] = bf16_lo(vw);
          x[2 * e + 1] = bf16_hi(vw);
        }
#pragma unroll
        for (int gi = 0; gi < GB; ++gi) {
          const float pw = ok ? __builtin_amdgcn_exp2f(sc[gi] - m[gi]) : 0.f;
          l[gi] += pw;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[gi][e] = fmaf(pw, x[e], o[gi][e]);
        }
      }
    }
  }

  // merge the row groups: first the GPW groups of each wavefront (lanes
  // that differ in the row-group bits), then the wavefronts through LDS
#pragma unroll
  for (int gi = 0; gi < GB; ++gi) {
    float mw = m[gi];
    for (int x = LPK; x < 64; x <<= 1) mw = fmaxf(mw, __shfl_xor(mw, x));
    const float a =
        m[gi] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[gi] - mw);
    float lw = l[gi] * a;
    for (int x = LPK; x < 64; x <<= 1) lw += __shfl_xor(lw, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float y = o[gi][e] * a;
      for (int x = LPK; x < 64; x <<= 1) y += __shfl_xor(y, x);
      o[gi][e] = y;
    }
    m[gi] = mw;
    l[gi] = lw;
  }
  if (lane < LPK) {
#pragma unroll
    for (int gi = 0; gi < GB; ++gi)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wave][gi * D + dch * 8 + e] = o[gi][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int gi = 0; gi < GB; ++gi) {
      red_ml[wave][gi] = m[gi];
      red_ml[wave][GB + gi] = l[gi];
    }
  }
  __syncthreads();
  for (int t = tid; t < nh * D; t += kThreads) {
    const int gi = t / D;
    const int d = t - gi * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) mx = fmaxf(mx, red_ml[w][gi]);
    float x = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = red_ml[w][gi];
      const float a = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mx);
      x = fmaf(a, red_o[w][t], x);
      lsum = fmaf(a, red_ml[w][GB + gi], lsum);
    }
    const size_t row = (size_t)(b * p.Hq + h0 + gi) * p.nsplit + s;
    p.ws_o[row * D + d] = x / lsum;
    if (d == 0) p.ws_lse[row] = (mx + log2f(lsum)) * 0.69314718055994531f;
  }
}

// One wavefront per (batch, query head); lane l owns columns l*CPL..+CPL-1.
template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void decode_combine_kernel(
    DecodeParams p) {
  constexpr int CPL = D / 64;
  const int r = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (r >= p.B * p.Hq) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int b = r / p.Hq;
  int lo, L, sk;
  key_range(p, b, lo, L, sk);
  const size_t row0 = (size_t)r * p.nsplit;
  uint16_t* orow = p.o + (size_t)r * D + lane * CPL;
  if (L <= lo && sk == 0) {  // no allowed key
#pragma unroll
    for (int e = 0; e < CPL; ++e) orow[e] = 0;
    if (lane == 0 && p.lse) p.lse[r] = -INFINITY;
    return;
  }
  // the splits the split kernel wrote: those holding an allowed key
  const int s0 = sk > 0 ? 0 : lo / kChunk;
  const int s1 = (L + kChunk - 1) / kChunk;
  auto live = [&](int s) {
    const int c0 = s * kChunk;
    return split_first_key(c0, min(c0 + kChunk, L), lo, sk) <
           min(c0 + kChunk, L);
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

int heads_per_block(int G) {
  if (G <= kMaxGB) return G;
  for (int gb = kMaxGB; gb > 1; --gb)
    if (G % gb == 0) return gb;
  return 1;
}

template <int D, int GB>
void launch_split(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((decode_split_kernel<D, GB>),
                     dim3(p.B * p.Hkv * p.nhc, p.nsplit), dim3(kThreads), 0, st,
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

int decode_max_keys() { return 65535 * kChunk; }

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
  p.sinks = pr.sinks;
  p.nsplit = (pr.Nk + kChunk - 1) / kChunk;
  p.c = pr.scale * 1.4426950408889634f;
  const size_t rows = (size_t)pr.B * pr.Hq * p.nsplit;
  p.ws_o = static_cast<float*>(ws);
  p.ws_lse = p.ws_o + rows * pr.d;
  const int ncomb = (pr.B * pr.Hq + kCombineWaves - 1) / kCombineWaves;
  if (pr.d == 128) {
    launch_split_d<128>(p, stream);
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(ncomb),
                       dim3(64 * kCombineWaves), 0, stream, p);
  } else {
    launch_split_d<64>(p, stream);
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(ncomb),
                       dim3(64 * kCombineWaves), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace miattn
