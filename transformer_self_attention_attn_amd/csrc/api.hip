// C-ABI layer of libmiattn: argument validation (host only, before any HIP
// call), dispatch to the kernels, the decode workspace and error reporting.
// The contract is documented in include/miattn.h.
#include "miattn.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Shared checks of attn_fwd and attn_fwd_f32.  No HIP call happens here.
int validate(const char* fn, const void* q, const void* k, const void* v,
             const void* o, const float* lse, int B, int Hq, int Hkv, int Nq,
             int Nk, int d, float scale, int causal, int window,
             int window_right, int sinks, bool one_sided) {
  if (!q || !k || !v || !o)
    return fail(MIATTN_ERR_INVALID, "%s: q, k, v and o must be non-null", fn);
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0)
    return fail(MIATTN_ERR_INVALID,
                "%s: sizes must be positive (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d "
                "d=%d)",
                fn, B, Hq, Hkv, Nq, Nk, d);
  if (Hq % Hkv != 0)
    return fail(MIATTN_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d",
                fn, Hq, Hkv);
  if (Nq > Nk)
    return fail(MIATTN_ERR_INVALID, "%s: Nq=%d exceeds Nk=%d", fn, Nq, Nk);
  if (window < 0 || window_right < 0 || sinks < 0)
    return fail(MIATTN_ERR_INVALID,
                "%s: window=%d, window_right=%d, sinks=%d: none may be "
                "negative", fn, window, window_right, sinks);
  if (!std::isfinite(scale))
    return fail(MIATTN_ERR_INVALID, "%s: scale is not finite", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned16(lse)))
    return fail(MIATTN_ERR_INVALID,
                "%s: q, k, v, o and lse must be 16-byte aligned", fn);
  if (d != 64 && d != 128)
    return fail(MIATTN_ERR_UNSUPPORTED, "%s: head dim d=%d (supported: 64, 128)",
                fn, d);
  if (one_sided && window > 0 && !causal)
    return fail(MIATTN_ERR_UNSUPPORTED,
                "%s: a window needs the causal mask (one-sided look-back)", fn);
  // index arithmetic bounds: element offsets are 64-bit, row and block
  // counts are 32-bit
  const long long qrows = (long long)B * Hq * Nq;
  const long long qblocks = (long long)B * Hq * ((Nq + 127) / 128);
  if (qrows > 0x7fffffffLL || qblocks > 0x7fffffffLL ||
      (long long)B * Hkv * Nk > 0x7fffffffLL)
    return fail(MIATTN_ERR_INVALID, "%s: problem too large for one launch",
                fn);
  return MIATTN_OK;
}

// ---- workspace of the decode and backward passes, one per device ---------
// The lock is held from the size check through the launch that uses the
// buffer, so a growth by another host thread (which frees the old buffer)
// cannot slip in between.  Growth calls hipFree and hipMalloc: the free
// waits for the device to finish the work still using the old buffer.
constexpr int kMaxDevices = 64;
std::mutex g_ws_mu;
void* g_ws[kMaxDevices] = {};
size_t g_ws_bytes[kMaxDevices] = {};

int current_device(int* dev) {
  const hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess)
    return fail(MIATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (*dev < 0 || *dev >= kMaxDevices)
    return fail(MIATTN_ERR_HIP, "device index %d out of range", *dev);
  return MIATTN_OK;
}

// Caller holds g_ws_mu.
int workspace_locked(size_t need, void** out) {
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != MIATTN_OK) return rc;
  hipError_t e;
  if (g_ws_bytes[dev] < need) {
    if (g_ws[dev]) {
      e = hipFree(g_ws[dev]);  // waits for work still using it
      g_ws[dev] = nullptr;
      g_ws_bytes[dev] = 0;
      if (e != hipSuccess)
        return fail(MIATTN_ERR_HIP, "hipFree: %s", hipGetErrorString(e));
    }
    e = hipMalloc(&g_ws[dev], need);
    if (e != hipSuccess) {
      g_ws[dev] = nullptr;
      (void)hipGetLastError();
      return fail(MIATTN_ERR_NOMEM, "workspace of %zu bytes: %s", need,
                  hipGetErrorString(e));
    }
    g_ws_bytes[dev] = need;
  }
  *out = g_ws[dev];
  return MIATTN_OK;
}

// Sequences whose whole extent is addressed by one 32-bit buffer resource
// (the backward and FP8 kernels): q/o rows of a (batch, head) and k/v rows,
// padded to whole 64-key tiles, must span less than 2^31 bytes.
int check_sequence_bytes(const char* fn, int Nq, int Nk, int d) {
  const long long lim = 1LL << 31;
  const long long nkp = ((long long)Nk + 63) / 64 * 64;
  if ((long long)Nq * d * 2 >= lim || nkp * d * 2 >= lim)
    return fail(MIATTN_ERR_UNSUPPORTED,
                "%s: one sequence of Nq=%d or Nk=%d rows at d=%d spans 2^31 "
                "bytes or more", fn, Nq, Nk, d);
  return MIATTN_OK;
}

miattn::Problem make_problem(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                             float scale, int causal, int window,
                             int window_right, int sinks,
                             const int* seqlens) {
  miattn::Problem p;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.d = d;
  p.scale = scale;
  p.causal = causal ? 1 : 0;
  // a query position lies in [-Nq, Nk) and a key in [0, Nk), so a window
  // of Nq + Nk or more keeps every key on its side and sinks beyond Nk add
  // nothing; clamping keeps the kernels' index arithmetic inside int
  const long long span = (long long)Nq + Nk;
  p.window = (int)std::min<long long>(window, span);
  p.window_right = (int)std::min<long long>(window_right, span);
  p.sinks = std::min(sinks, Nk);
  p.seqlens = seqlens;
  return p;
}

// bf16 dispatch shared by attn_fwd and attn_fwd_masked (arguments checked)
int run_bf16(const char* fn, const void* q, const void* k, const void* v,
             void* o, float* lse, const miattn::Problem& p, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  int rc;
  // the prefill kernel reads a head's query rows through one 32-bit buffer
  // resource, with 32-bit byte offsets: they must span less than 2^31 bytes
  // (the decode kernel's offsets are 64-bit)
  if (!miattn::decode_takes(p) && (long long)p.Nq * p.d * 2 >= (1LL << 31))
    return fail(MIATTN_ERR_UNSUPPORTED,
                "%s: one sequence of Nq=%d query rows at d=%d spans 2^31 "
                "bytes or more", fn, p.Nq, p.d);
  if (miattn::decode_takes(p)) {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    void* ws = nullptr;
    rc = workspace_locked(miattn::decode_workspace_bytes(p), &ws);
    if (rc != MIATTN_OK) return rc;
    e = miattn::launch_decode_bf16(q, k, v, o, lse, p, ws, st);
  } else {
    e = miattn::launch_prefill_bf16(q, k, v, o, lse, p, st);
  }
  if (e != hipSuccess)
    return fail(MIATTN_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return MIATTN_OK;
}

int run_f32(const char* fn, const float* q, const float* k, const float* v,
            float* o, float* lse, const miattn::Problem& p, void* stream) {
  const hipError_t e = miattn::launch_attn_f32(
      q, k, v, o, lse, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MIATTN_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return MIATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             int causal, int window, const int* seqlens, void* stream) {
  const int rc = validate("attn_fwd", q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d,
                          scale, causal, window, 0, 0, true);
  if (rc != MIATTN_OK) return rc;
  return run_bf16("attn_fwd", q, k, v, o, lse,
                  make_problem(B, Hq, Hkv, Nq, Nk, d, scale, causal, window,
                               0, 0, seqlens),
                  stream);
}

int attn_fwd_masked(const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                    float scale, int causal, int window_left,
                    int window_right, int sinks, const int* seqlens,
                    void* stream) {
  const int rc = validate("attn_fwd_masked", q, k, v, o, lse, B, Hq, Hkv, Nq,
                          Nk, d, scale, causal, window_left, window_right,
                          sinks, false);
  if (rc != MIATTN_OK) return rc;
  return run_bf16("attn_fwd_masked", q, k, v, o, lse,
                  make_problem(B, Hq, Hkv, Nq, Nk, d, scale, causal,
                               window_left, window_right, sinks, seqlens),
                  stream);
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                 float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, int window, const int* seqlens,
                 void* stream) {
  const int rc = validate("attn_fwd_f32", q, k, v, o, lse, B, Hq, Hkv, Nq, Nk,
                          d, scale, causal, window, 0, 0, true);
  if (rc != MIATTN_OK) return rc;
  return run_f32("attn_fwd_f32", q, k, v, o, lse,
                 make_problem(B, Hq, Hkv, Nq, Nk, d, scale, causal, window, 0,
                              0, seqlens),
                 stream);
}

int attn_fwd_masked_f32(const float* q, const float* k, const float* v,
                        float* o, float* lse, int B, int Hq, int Hkv, int Nq,
                        int Nk, int d, float scale, int causal,
                        int window_left, int window_right, int sinks,
                        const int* seqlens, void* stream) {
  const int rc = validate("attn_fwd_masked_f32", q, k, v, o, lse, B, Hq, Hkv,
                          Nq, Nk, d, scale, causal, window_left, window_right,
                          sinks, false);
  if (rc != MIATTN_OK) return rc;
  return run_f32("attn_fwd_masked_f32", q, k, v, o, lse,
                 make_problem(B, Hq, Hkv, Nq, Nk, d, scale, causal,
                              window_left, window_right, sinks, seqlens),
                 stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* lse, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             int causal, int window_left, int window_right, int sinks,
             const int* seqlens, void* stream) {
  const char* fn = "attn_bwd";
  int rc = validate(fn, q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                    window_left, window_right, sinks, false);
  if (rc != MIATTN_OK) return rc;
  if (!dout || !lse || !dq || !dk || !dv)
    return fail(MIATTN_ERR_INVALID,
                "%s: dout, lse, dq, dk and dv must be non-null", fn);
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(MIATTN_ERR_INVALID,
                "%s: dout, dq, dk and dv must be 16-byte aligned", fn);
  rc = check_sequence_bytes(fn, Nq, Nk, d);
  if (rc != MIATTN_OK) return rc;
  const miattn::Problem p =
      make_problem(B, Hq, Hkv, Nq, Nk, d, scale, causal, window_left,
                   window_right, sinks, seqlens);
  std::lock_guard<std::mutex> lock(g_ws_mu);
  void* ws = nullptr;
  rc = workspace_locked(miattn::bwd_workspace_bytes(p), &ws);
  if (rc != MIATTN_OK) return rc;
  const hipError_t e =
      miattn::launch_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, p, ws,
                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MIATTN_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return MIATTN_OK;
}

int attn_fp8_quantize(const void* q, const void* k, const void* v, int B,
                      int Hq, int Hkv, int Nq, int Nk, int d,
                      const int* seqlens, const signed char* signs,
                      int per_tensor, void* q8, float* sq, void* k8,
                      float* sk, void* v8t, float* sv, void* stream) {
  const char* fn = "attn_fp8_quantize";
  // shape checks as for the forward (q stands in for o)
  int rc = validate(fn, q, k, v, q, nullptr, B, Hq, Hkv, Nq, Nk, d, 1.0f, 0,
                    0, 0, 0, false);
  if (rc != MIATTN_OK) return rc;
  if (!q8 || !sq || !k8 || !sk || !v8t || !sv)
    return fail(MIATTN_ERR_INVALID,
                "%s: q8, sq, k8, sk, v8t and sv must be non-null", fn);
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) ||
      (reinterpret_cast<uintptr_t>(sq) | reinterpret_cast<uintptr_t>(sk) |
       reinterpret_cast<uintptr_t>(sv)) & 3u)
    return fail(MIATTN_ERR_INVALID,
                "%s: q8, k8, v8t must be 16-byte aligned, the scales 4-byte",
                fn);
  rc = check_sequence_bytes(fn, Nq, Nk, d);
  if (rc != MIATTN_OK) return rc;
  const miattn::Problem p =
      make_problem(B, Hq, Hkv, Nq, Nk, d, 1.0f, 0, 0, 0, 0, seqlens);
  const hipError_t e = miattn::launch_fp8_quantize(
      q, k, v, p, signs, per_tensor, q8, sq, k8, sk, v8t, sv,
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MIATTN_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return MIATTN_OK;
}

int attn_fwd_fp8(const void* q8, const float* sq, const void* k8,
                 const float* sk, const void* v8t, const float* sv, void* o,
                 float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int rotated, int causal, int window_left,
                 int window_right, int sinks, const int* seqlens,
                 void* stream) {
  const char* fn = "attn_fwd_fp8";
  int rc = validate(fn, q8, k8, v8t, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                    causal, window_left, window_right, sinks, false);
  if (rc != MIATTN_OK) return rc;
  if (!sq || !sk || !sv)
    return fail(MIATTN_ERR_INVALID, "%s: sq, sk and sv must be non-null", fn);
  if ((reinterpret_cast<uintptr_t>(sq) | reinterpret_cast<uintptr_t>(sk) |
       reinterpret_cast<uintptr_t>(sv)) & 3u)
    return fail(MIATTN_ERR_INVALID, "%s: the scales must be 4-byte aligned",
                fn);
  rc = check_sequence_bytes(fn, Nq, Nk, d);
  if (rc != MIATTN_OK) return rc;
  const miattn::Problem p =
      make_problem(B, Hq, Hkv, Nq, Nk, d, scale, causal, window_left,
                   window_right, sinks, seqlens);
  const hipError_t e = miattn::launch_fwd_fp8(
      q8, sq, k8, sk, v8t, sv, o, lse, p, rotated,
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(MIATTN_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return MIATTN_OK;
}

const char* attn_last_error(void) { return g_err; }

void attn_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (int dev = 0; dev < kMaxDevices; ++dev) {
    if (!g_ws[dev]) continue;
    if (hipSetDevice(dev) == hipSuccess) (void)hipFree(g_ws[dev]);
    g_ws[dev] = nullptr;
    g_ws_bytes[dev] = 0;
  }
  if (have_cur) (void)hipSetDevice(cur);
}

}  // extern "C"
