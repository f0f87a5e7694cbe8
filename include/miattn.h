/*
 * libmiattn: forward multi-head scaled dot-product attention on gfx950.
 *
 *   O = softmax(scale * Q K^T + mask) V,    lse = log sum exp(scale * Q K^T + mask)
 *
 * The operation is the one stated on the pages this library follows:
 *  - score Q K^T / sqrt(D) and Softmax(score) V: "SpAtten: Efficient Sparse
 *    Attention Architecture with Cascade Token and Head Pruning" (review page),
 *    Background - Attention Mechanism; probability p_i = exp(s_i)/sum_j exp(s_j)
 *    in its Algorithm Optimization section D (Progressive Quantization);
 *  - scaled dot-product with sqrt(d_k), softmax weights, weighted sum of V, the
 *    padding mask (-inf on pad tokens) and the look-ahead mask (self and earlier
 *    tokens only): the self-attention explainer page (palettepath-it), sections
 *    on score scaling, softmax normalisation, masking, multi-head attention;
 *  - local-window attention (each token looks at its neighbours) and
 *    variable-length padding: the O(n^2) tutorial page (devhandbook),
 *    "Local Window Attention" and Example 7;
 *  - grouped-query and sliding-window attention as named variants:
 *    "Attentions Under the Microscope" summary page, Methodology;
 *  - the problem statement Q, K, V in R^{N x d} -> O: the FlashAttention-3
 *    review page (deepmi.me), input data of the core algorithm;
 *  - the one-token generation step against a growing K/V cache: the SpAtten
 *    review, Background - Attention-Based NLP Models (generation stage), and
 *    its evaluation setting of new tokens after a prompt (EVALUATION);
 *  - encoder-decoder (cross) attention, decoder queries against the encoder's
 *    keys and values: the self-attention explainer page, decoder stack.
 *
 * Layout (all buffers contiguous, innermost dimension last, the
 * [batch, heads, n, d] order of the tutorial page's SDPA example):
 *   q, o : [B, Hq,  Nq, d]      k, v : [B, Hkv, Nk, d]
 *   lse  : [B, Hq,  Nq]  float32, natural log, scale applied
 *   seqlens : [B] int32 valid key lengths (right padding), or NULL = all Nk
 *
 * Semantics (the readings taken where the pages are silent):
 *   G = Hq / Hkv; query head h reads K/V head h / G (contiguous groups).
 *   L_b = clamp(seqlens[b], 0, Nk).  If Nq == Nk the first L_b query rows are
 *   live and row i sits at position i.  If Nq < Nk all Nq rows are live and
 *   they are the last Nq positions of the sequence: row i sits at position
 *   L_b - Nq + i ("bottom-right"; with Nq == 1 the single query is the last
 *   token and sees its own key; a row whose position is negative sees no key
 *   under the causal mask).  causal == 0 with Nq != Nk is cross-attention.
 *   Query row i may attend to key j iff i is live, j < L_b,
 *   (causal == 0 or j <= pos(i)) and (window <= 0 or pos(i) - j < window).
 *   Masked scores are excluded exactly (-inf), never a finite penalty.
 *   A row with no allowed key (dead padding rows included) gets O = 0 and
 *   lse = -inf.  Padded K/V/Q contents are never read into a result; they may
 *   hold NaN.
 *
 * Ownership: every pointer is a device pointer owned by the caller; the
 * library writes only its outputs (o and lse; dq, dk and dv for attn_bwd).
 *
 * Workspace: three paths keep partial results in a library-owned device
 * buffer, one per device: the decode step (Nq == 1), short chunks
 * (1 < Nq < Nk with (Hq / Hkv) * Nq <= 16, which run on the decode
 * kernels), and attn_bwd.  The buffer is allocated on a path's first call
 * and grown when a larger problem arrives; attn_release() frees it.
 * Growth calls hipFree and hipMalloc, and hipFree waits for the whole device
 * to finish: a call that grows the workspace synchronises the device.  Every
 * other call is asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream) and never synchronises; a caller that must not synchronise makes
 * one call of its largest size first.  With the workspace at its size, a
 * call is kernel launches on `stream` only, so it may be captured into a
 * HIP graph and replayed.  The
 * library holds a lock from the size check through the launch, so calls
 * from several host threads never free a buffer a queued launch still
 * names; but all workspace users on one device share the one buffer, so
 * their kernels must not overlap: issue them on one stream, or order the
 * streams.
 *
 * Run-time tail: a causal prefill (attn_fwd, attn_fwd_masked with no left
 * window) or attn_fwd_fp8 of at least three rounds of the chip's workgroup
 * slots takes its lightest query blocks from a device-wide ticket counter,
 * one counter set per call from a ring of 64 per device (a captured graph
 * keeps the set of its capture); the call's last workgroup to take a ticket
 * zeroes the set.  Such calls on one device whose kernels overlap in time
 * and hold the same set would race, so no more than 64 of them may run at
 * once on one device.
 *
 * Errors: the return value is a status.  Argument checks run on the host
 * before any HIP call, so they are testable without a GPU.  No call aborts or
 * throws.  attn_last_error() describes the most recent non-OK status of the
 * calling thread.
 */
#ifndef MIATTN_H
#define MIATTN_H

#ifdef __cplusplus
extern "C" {
#endif

enum miattn_status {
  MIATTN_OK = 0,
  MIATTN_ERR_INVALID = -1,      /* null pointer, size <= 0, Hq % Hkv != 0,
                                   Nq > Nk, window, window_right or sinks
                                   < 0, non-finite scale,
                                   pointer not 16-byte aligned, size overflow
                                   (B*Hq*Nq or B*Hkv*Nk above 2^31 - 1) */
  MIATTN_ERR_UNSUPPORTED = -2,  /* d not in {64, 128}; attn_fwd(_f32):
                                   window > 0 without causal; attn_bwd and
                                   the FP8 calls: one sequence (Nq rows, or
                                   Nk rows padded to 64, of d bf16) spanning
                                   2^31 bytes or more; attn_fwd(_masked)
                                   calls that take the prefill kernel (every
                                   call but Nq == 1 and short chunks): Nq
                                   rows of d bf16 spanning 2^31 bytes or
                                   more */
  MIATTN_ERR_HIP = -3,          /* a HIP runtime call or launch failed */
  MIATTN_ERR_NOMEM = -4         /* the workspace could not be grown */
};

/* bf16 q, k, v, o (raw 16-bit bfloat16 storage); float32 lse (may be NULL:
 * not written); int32 seqlens on the device (may be NULL).  Nq > 1 runs the
 * tiled MFMA kernel (prefill, chunked prefill, cross-attention); Nq == 1 runs
 * the split-K decode kernel followed by the log-sum-exp combine kernel. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             int causal, int window, const int* seqlens, void* stream);

/* Same contract with float32 q, k, v, o; fp32 arithmetic end to end. */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                 float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, int window, const int* seqlens,
                 void* stream);

/* attn_fwd with the window read on both sides and sink keys: the O(n^2)
 * tutorial page's local window (Local Window Attention strategy: a token
 * looks only at nearby tokens, on either side), and the attention sink that
 * the self-attention explainer page names in its roadmap (data-efficient
 * attention design) as a way to manage long context windows: the first keys
 * stay visible to every row whatever the window.  Query row i at
 * position pos(i) may attend to key j iff i is live, j < L_b,
 * (causal == 0 or j <= pos(i)) and
 *   ( (window_left  <= 0 or pos(i) - j < window_left) and
 *     (window_right <= 0 or j - pos(i) < window_right) )  or  j < sinks.
 * window_left is attn_fwd's window; a limit <= 0 is no limit.  Unlike
 * attn_fwd, a window without the causal mask is accepted (a two-sided
 * neighbourhood).  attn_fwd(..., window, ...) equals
 * attn_fwd_masked(..., window, 0, 0, ...).  Errors as attn_fwd, plus
 * MIATTN_ERR_INVALID for a negative window_right or sinks. */
int attn_fwd_masked(const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                    float scale, int causal, int window_left,
                    int window_right, int sinks, const int* seqlens,
                    void* stream);

/* attn_fwd_masked with float32 q, k, v, o. */
int attn_fwd_masked_f32(const float* q, const float* k, const float* v,
                        float* o, float* lse, int B, int Hq, int Hkv, int Nq,
                        int Nk, int d, float scale, int causal,
                        int window_left, int window_right, int sinks,
                        const int* seqlens, void* stream);

/* Backward pass (bf16): the gradients dq = dL/dq, dk = dL/dk, dv = dL/dv of a
 * scalar loss L given dout = dL/do, for the function attn_fwd_masked computes
 * with the same arguments.  The FlashAttention-3 review page names this pass
 * and its outputs (about 2.5 times the forward FLOPs) without its equations;
 * the gradient is the exact one of the forward definition, by the chain rule:
 *   p_ij = exp(scale q_i.k_j - lse_i) on allowed pairs (else 0),
 *   dv_j = sum_i p_ij dout_i,  ds_ij = p_ij (dout_i.v_j - dout_i.o_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 * with dk, dv of a K/V head summed over its Hq/Hkv query heads.
 * Inputs: q, k, v as for attn_fwd_masked; o and lse (float32, required) the
 * outputs attn_fwd / attn_fwd_masked gave for them; dout like o.  Outputs:
 * dq like q, dk and dv like k (bf16, fully written: rows of dead queries,
 * padding keys and keys no row may see get 0).  Accumulation is fp32; P and
 * dS enter their products rounded to bf16.  Errors as attn_fwd_masked, plus
 * MIATTN_ERR_INVALID for a null or misaligned dout, lse, dq, dk or dv. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* lse, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             int causal, int window_left, int window_right, int sinks,
             const int* seqlens, void* stream);

/* FP8 path (the FlashAttention-3 review page's FP8 sections: E4M3 operands,
 * block quantization, incoherent processing).
 *
 * attn_fp8_quantize: bf16 q, k, v (layouts and seqlens as for attn_fwd) to
 * E4M3 codes and float32 block scales.  With `signs` (device pointer to d
 * entries +1/-1, or NULL) Q and K are first multiplied by M = diag(signs) H,
 * H the Sylvester Hadamard matrix with entries +-1 (so Q'' K''^T = d Q K^T;
 * pass rotated = 1 to attn_fwd_fp8); V is never rotated.  Each 64-row block
 * of a (batch, head) gets scale s = amax / 448 (amax over its valid rows; 0
 * for an empty block) and codes E4M3(x * 448 / amax), rounded to nearest
 * even, in float32.  per_tensor = 1 instead uses one amax per tensor (the
 * baseline of the page's accuracy comparison).  Outputs (device, caller
 * owned; Nkp = Nk rounded up to 64):
 *   q8  [B][Hq][Nq][d] bytes           sq [B][Hq][ceil(Nq/64)] float
 *   k8  [B][Hkv][Nkp][d] bytes         sk [B][Hkv][Nkp/64] float
 *   v8t [B][Hkv][Nkp/64][d][64] bytes  sv [B][Hkv][Nkp/64] float
 * (v8t holds each 64-key tile of V transposed).  Rows past the valid length
 * and dead query rows hold code 0.  q8, k8, v8t 16-byte aligned.
 *
 * attn_fwd_fp8: attention of the dequantized operands, o (bf16) and lse as
 * attn_fwd_masked computes them from q, k, v, with the same mask arguments;
 * `scale` is the caller's softmax scale (divided by d inside when rotated).
 * Both products run on FP8 matrix cores with fp32 accumulation; the
 * probabilities enter the second product as E4M3 (times 256 and the tile's
 * V scale relative to the head's largest).  Errors as attn_fwd_masked, plus
 * MIATTN_ERR_INVALID for null or misaligned quantized buffers. */
int attn_fp8_quantize(const void* q, const void* k, const void* v, int B,
                      int Hq, int Hkv, int Nq, int Nk, int d,
                      const int* seqlens, const signed char* signs,
                      int per_tensor, void* q8, float* sq, void* k8,
                      float* sk, void* v8t, float* sv, void* stream);

int attn_fwd_fp8(const void* q8, const float* sq, const void* k8,
                 const float* sk, const void* v8t, const float* sv, void* o,
                 float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int rotated, int causal, int window_left,
                 int window_right, int sinks, const int* seqlens,
                 void* stream);

/* Message for the calling thread's most recent non-OK status ("" if none).
 * The pointer stays valid until the thread's next failing call. */
const char* attn_last_error(void);

/* Frees the library-owned workspace on every device that has one.
 * The caller must ensure no call that uses it (see Workspace above) is
 * still running. */
void attn_release(void);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
