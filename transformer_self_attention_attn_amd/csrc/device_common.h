// Device helpers shared by the backward and FP8 kernels: the row-position
// and mask arithmetic of the boundary's semantics, the MFMA row order, the
// direct-to-LDS buffer load, waits and barriers, wave reductions and the
// XCD-aware block order.  Internal; not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "lane_layout.h"

typedef int miattn_i32x4 __attribute__((ext_vector_type(4)));

// The direct-to-LDS buffer load (buffer_load_dword* ... lds), declared by
// its intrinsic name with the resource as four plain ints: written with the
// resource-type builtins, kernels using it lost their host-side launch stubs
// in this compiler.
__device__ void miattn_buffer_load_lds(
    miattn_i32x4 rsrc, __attribute__((address_space(3))) void* lds, int size,
    int voffset, int soffset, int offset,
    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
// The 16-byte buffer load into registers, declared the same way: a lane's
// bytes at or past the resource's end read as zeros.
__device__ miattn_i32x4 miattn_buffer_load_b128(
    miattn_i32x4 rsrc, int voffset, int soffset,
    int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");

namespace miattn {
namespace dev {

template <int N>
using ic = std::integral_constant<int, N>;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(ic<I>());
    static_for<I + 1, N>(f);
  }
}

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies
constexpr int kBig = 1 << 30;

// Valid length and row positions of batch b: rows i < Lq are live and row i
// sits at position i + off (Nq == Nk: the first L rows; otherwise the last Nq
// positions of the sequence).
struct Seq {
  int L, Lq, off;
};
__device__ inline Seq seq_of(const int* seqlens, int Nq, int Nk, int b) {
  int L = Nk;
  if (seqlens) {
    L = seqlens[b];
    L = L < 0 ? 0 : (L > Nk ? Nk : L);
  }
  const int Lq = (Nq == Nk) ? L : Nq;
  return {L, Lq, L - Lq};
}

// Keys of a row at position pos: those below hc (valid length; pos + 1 under
// the causal mask), and of them the window keys [lo, hw) (left limit
// pos - j < wl, right limit j - pos < wr, each off when 0) and the sink keys
// [0, sk).  All zero for a dead row.
struct RowKeys {
  int hc, hw, lo, sk;
};
__device__ inline RowKeys keys_of_row(const Seq& s, int causal, int wl, int wr,
                                      int sinks, bool live, int pos) {
  if (!live) return {0, 0, 0, 0};
  RowKeys r;
  r.hc = max(0, causal ? min(s.L, pos + 1) : s.L);
  r.hw = wr > 0 ? max(0, min(r.hc, pos + wr)) : r.hc;
  r.lo = wl > 0 ? max(0, pos - wl + 1) : 0;
  r.sk = min(sinks, r.hc);
  return r;
}

// Query rows [lo, hi) that may see key j (empty when lo >= hi): pos >= j
// under the causal mask and, unless j is a sink key, j - wr < pos < j + wl.
__device__ inline void rows_of_key(const Seq& s, int causal, int wl, int wr,
                                   int sinks, int j, int& lo, int& hi) {
  if (j >= s.L) {
    lo = s.Lq;
    hi = 0;
    return;
  }
  int plo = causal ? j : -kBig;
  int phi = kBig;
  if (j >= sinks) {
    if (wr > 0) plo = max(plo, j - wr + 1);
    if (wl > 0) phi = j + wl;
  }
  lo = max(0, plo - s.off);
  hi = min(s.Lq, phi - s.off);
}

// Row of a 32-row MFMA A-operand block that holds tile row m: with this order
// the 32x32 accumulator gives lane group g (lanes 32g .. 32g+31) the 16
// consecutive tile rows g*16 .. g*16+15 of each 32-row block.
__device__ inline int mfma_row(int m) { return lanes::mfma_row(m); }

// Buffer resource over `bytes` bytes at `base` (stride 0, 32-bit data
// format): a load at or past the end reads zeros.
__device__ inline miattn_i32x4 rows_rsrc(const void* base, int bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  miattn_i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;
  return r;
}

// Waits for every vector-memory load of this wave; other counters untouched.
__device__ inline void wait_vm0() { __builtin_amdgcn_s_waitcnt(0xF70); }

// Waits until at most n (0 .. 15, wave-uniform) vector-memory loads of this
// wave are outstanding (vmcnt is bits 3:0 here).
__device__ inline void wait_vmcnt_rt(int n) {
  switch (n) {
#define MIATTN_DEV_VM(N)                      \
  case N:                                     \
    __builtin_amdgcn_s_waitcnt(0xF70 | (N)); \
    break;
    MIATTN_DEV_VM(1) MIATTN_DEV_VM(2) MIATTN_DEV_VM(3) MIATTN_DEV_VM(4)
    MIATTN_DEV_VM(5) MIATTN_DEV_VM(6) MIATTN_DEV_VM(7) MIATTN_DEV_VM(8)
    MIATTN_DEV_VM(9) MIATTN_DEV_VM(10) MIATTN_DEV_VM(11) MIATTN_DEV_VM(12)
    MIATTN_DEV_VM(13) MIATTN_DEV_VM(14) MIATTN_DEV_VM(15)
#undef MIATTN_DEV_VM
    default:
      __builtin_amdgcn_s_waitcnt(0xF70);
  }
}

// Workgroup barrier without a memory fence (loads are awaited explicitly;
// the clobber keeps the compiler from moving memory accesses across it).
__device__ inline void barrier_nofence() {
  asm volatile("s_barrier" ::: "memory");
}

__device__ inline float wave_maxf(float x) {
  for (int s = 32; s > 0; s >>= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}
__device__ inline int wave_imin(int x) {
  for (int s = 32; s > 0; s >>= 1) x = min(x, __shfl_xor(x, s));
  return x;
}
__device__ inline int wave_imax(int x) {
  for (int s = 32; s > 0; s >>= 1) x = max(x, __shfl_xor(x, s));
  return x;
}

// Block index -> logical block: consecutive logical blocks share an XCD (and
// its L2), so blocks of one (batch, K/V head) group meet in one cache.
__device__ inline int xcd_block(int bid, int n) {
  const int xcd = bid % kXcds;
  const int slot = bid / kXcds;
  const int per = n / kXcds;
  const int rem = n % kXcds;
  return xcd * per + min(xcd, rem) + slot;
}

}  // namespace dev
}  // namespace miattn
