// Internal interface between the C-ABI layer (api.hip) and the kernel files.
// Not installed; callers use include/miattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace miattn {

// One attention problem, already validated by the C-ABI layer.
struct Problem {
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int window;        // left limit: pos - window < j (0 = none)
  int window_right;  // right limit: j < pos + window_right (0 = none)
  int sinks;         // keys j < sinks allowed whatever the window says
  const int* seqlens;  // device pointer or nullptr
};

// Tiled bf16 MFMA prefill: Nq == Nk, and 1 < Nq < Nk (chunks against a
// cache, cross-attention) where decode_takes is false.
hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v,
                               void* o, float* lse, const Problem& p,
                               hipStream_t stream);

// Split-K bf16 decode and its log-sum-exp combine: Nq == 1, and short chunks
// 1 < Nq < Nk whose rows fit a few 16-column blocks (decode_takes).  `ws`
// must hold decode_workspace_bytes(p) bytes.
bool decode_takes(const Problem& p);
size_t decode_workspace_bytes(const Problem& p);
hipError_t launch_decode_bf16(const void* q, const void* k, const void* v,
                              void* o, float* lse, const Problem& p, void* ws,
                              hipStream_t stream);

// bf16 backward: dQ, dK, dV from q, k, v, o, dO and the forward lse.  `ws`
// must hold bwd_workspace_bytes(p) bytes.
size_t bwd_workspace_bytes(const Problem& p);
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse,
                           void* dq, void* dk, void* dv, const Problem& p,
                           void* ws, hipStream_t stream);

// FP8 path: quantization (bf16 q, k, v -> E4M3 codes and block scales, Q and
// K rotated when `signs` is non-null) and the forward kernel on the codes.
hipError_t launch_fp8_quantize(const void* q, const void* k, const void* v,
                               const Problem& p, const signed char* signs,
                               int per_tensor, void* q8, float* sq, void* k8,
                               float* sk, void* v8t, float* sv,
                               hipStream_t stream);
hipError_t launch_fwd_fp8(const void* q8, const float* sq, const void* k8,
                          const float* sk, const void* v8t, const float* sv,
                          void* o, float* lse, const Problem& p, int rotated,
                          hipStream_t stream);

// fp32 path (any 1 <= Nq <= Nk).
hipError_t launch_attn_f32(const float* q, const float* k, const float* v,
                           float* o, float* lse, const Problem& p,
                           hipStream_t stream);

}  // namespace miattn
