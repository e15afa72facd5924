/*
 * hr.h -- C ABI of libhr: batched prefill of a Qwen3-style decoder stack that
 * feeds a multi-codebook audio head, and the head's delayed-codebook step, on
 * one AMD Instinct MI355X (gfx950).
 *
 * What the calls compute (sources cited by page title and section):
 *  - "Stabilize Higgs Audio termination and prefill" (FlashRT pull request 141),
 *    Summary: the batched prefill is embedding lookup, projection GEMMs, q/k
 *    norm + RoPE and KV writes; a delayed-codebook helper does per-frame
 *    argmax, delay handling and codebook-embedding accumulation; the delayed
 *    EOC check must cover every codebook (Root cause); FP8 activation scales
 *    are static, taken once from a fixed calibration prompt.
 *  - flashrt-structures 0.2.0, prefill_tower/fp8_chain.py, module docstring and
 *    the per-call `run`: RMSNorm -> merged QKV GEMM -> split + RoPE + KV cache
 *    -> attention over exactly the used keys -> output projection -> fused
 *    residual + RMSNorm -> merged gate/up GEMM -> activation -> down GEMM;
 *    static per-tensor activation scales `amax / FP8_MAX`, GEMM alpha =
 *    activation scale x weight scale; a raw-pointer GEMM entry
 *    `(x, w, out, M, N, K, alpha, beta, stream)` is the precedent for this ABI.
 *  - "feat(higgs-audio): add checkpoint loading and validation foundation"
 *    (pegainfer pull request 864), Summary: the backbone's final hidden feeds
 *    the audio-head projection.
 *  - vLLM-Omni pull request 8226 (Higgs Audio v3 on Model Runner V2), Purpose:
 *    a launch bound smaller than the longest query silently breaks attention,
 *    so bounds are checked, never assumed (HR_EBOUND).
 *
 * Conventions for every call:
 *  - All tensors are row-major (packed weights: the layout of hr_pack_weight)
 *    and live in device memory owned by the caller; the library never
 *    allocates or frees device memory, and reads none on the host except the
 *    one-word range check of hr_pack_weight.
 *  - bf16 tensors are passed as `const void*` (IEEE bfloat16 bit patterns);
 *    e4m3 tensors as OCP FP8 E4M3 (e4m3fn) bytes.
 *  - Every check runs on the host before the first launch; a call that
 *    returns a non-OK status has enqueued nothing (hr_pack_weight's range
 *    check, which needs the data, is the exception: it reports after the
 *    pack).  Work is enqueued on `stream` in order; the call returns without
 *    synchronising (hr_pack_weight does synchronise).
 *  - Device pointers must be 16-byte aligned (HR_EALIGN otherwise).
 *  - hr_last_error() returns a thread-local message for the last failure.
 */
#ifndef HR_H
#define HR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HR_OK = 0,
  HR_EINVAL = -1,        /* null pointer, bad size, cu_seqlens not monotone, ... */
  HR_EUNSUPPORTED = -2,  /* shape outside what the kernels implement            */
  HR_ECAPACITY = -3,     /* start_pos + len > capacity, cache_slot >= n_slots    */
  HR_EBOUND = -4,        /* max_seqlen < a sequence length, used_keys > length   */
  HR_EWORKSPACE = -5,    /* workspace smaller than hr_workspace_bytes()          */
  HR_EALIGN = -6,        /* device pointer not 16-byte aligned                   */
  HR_EHIP = -7           /* a HIP launch error                                   */
} hr_status;

/* Number formats.  Weights: HR_BF16, HR_FP8_E4M3, HR_MXFP4, HR_F16_PACKED.
 * HR_F16 (IEEE binary16) names the activations of the bf16-weight band where a
 * step entry of hr_ops.h takes an activation type.  HR_F16_PACKED: bf16
 * weights prepared once by hr_pack_weight (fp16 values in a slab-major
 * layout); a layer of them computes exactly what the HR_BF16 layer computes. */
typedef enum {
  HR_BF16 = 0, HR_FP8_E4M3 = 1, HR_MXFP4 = 2, HR_F16 = 3, HR_F16_PACKED = 4,
  /* range markers, never valid arguments: they give the type the whole int32
     range, so any value a caller passes is a value of the type that the
     checks reject (HR_EINVAL), not undefined behaviour */
  HR_WTYPE_RANGE_MIN_ = INT32_MIN, HR_WTYPE_RANGE_MAX_ = INT32_MAX
} hr_wtype;

/* Shapes of the decoder.  Supported: head_dim in {64, 128};
 * n_q_heads / n_kv_heads in {1, 2, 4}; hidden, ffn multiples of 64. */
typedef struct {
  int32_t hidden;      /* D */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv */
  int32_t head_dim;    /* d */
  int32_t ffn;         /* F (SwiGLU width) */
  int32_t n_layers;    /* L (hr_prefill_stack) */
  float rope_theta;    /* RoPE base, e.g. 1e6 */
  float rms_eps;       /* RMSNorm epsilon, e.g. 1e-6 */
  int32_t causal;      /* 1: query i sees cache positions [0, start_pos+i];
                          0: every query sees [0, used_keys[s]) and rows
                             i >= used_keys[s] are trailing pads            */
} hr_dims;

/* One decoder layer: device pointers, weights row-major [out, in] (packed
 * layers: the layout of hr_pack_weight).
 *  bf16:  w_* are bf16.  The activations between the kernels are fp16 (the
 *         norm outputs, the attention output, the SwiGLU product; 11-bit
 *         significand), the merged QKV rows fp32, the residual fp32 and the KV
 *         cache bf16; the GEMMs and attention run fp16 MFMAs (weights and
 *         cache rows converted exactly in registers) with fp32 accumulation.
 *         bf16 activations would hold the layer only to about 4e-2 of the
 *         exact result on 4B-class shapes (the bf16 storage points alone), the
 *         fp16 ones to about 1e-2, at the same MFMA rate.
 *  FP8:   w_* are e4m3 codes with per-output-channel fp32 scales ws_* so that
 *         W[n, k] ~= ws[n] * e4m3(w[n, k]); as_* are the static per-tensor
 *         activation scales (host floats): the GEMM input x is quantised as
 *         e4m3(x / as) and the product is rescaled by as * ws[n].
 *  MXFP4: the band of flashrt-structures 0.2.0 prefill_tower/fp8_chain.py (the
 *         FP4 band table: O and the FFN pair in 4-bit with dynamic block
 *         scales, QKV unchanged) in gfx950's OCP MX form (hr_ops.h): w_qkv is
 *         bf16; w_o, w_gu, w_down are E2M1 codes [N, K/2] packed by
 *         hr_quantize_mxfp4 with the AWQ scales of their input channels
 *         (and 1/s of the down projection on the up rows), their block scales
 *         in mx_*_s (slab-interleaved, ld = N); awq_inv_o / awq_inv_gu are the
 *         1/s vectors applied to the attention output and the FFN input before
 *         they are quantised per row (NULL: 1).  D a multiple of 256, Hq d and
 *         F multiples of 128.
 * Row order of w_qkv: q heads, then k heads, then v heads ([(Hq+2Hkv)d, D]).
 * Row order of w_gu: the gate projection, then the up projection ([2F, D]). */
typedef struct {
  hr_wtype wtype;
  const void* in_norm_w;    /* bf16 [D] */
  const void* post_norm_w;  /* bf16 [D] */
  const void* q_norm_w;     /* bf16 [d] */
  const void* k_norm_w;     /* bf16 [d] */
  const void* w_qkv;        /* [(Hq+2Hkv)d, D] */
  const void* w_o;          /* [D, Hq d] */
  const void* w_gu;         /* [2F, D] */
  const void* w_down;       /* [D, F] */
  const float* ws_qkv;      /* FP8 only: [(Hq+2Hkv)d] */
  const float* ws_o;        /* FP8 only: [D] */
  const float* ws_gu;       /* FP8 only: [2F] */
  const float* ws_down;     /* FP8 only: [D] */
  float as_qkv, as_o, as_gu, as_down;  /* FP8 only, > 0 */
  const uint8_t* mx_o_s;     /* MXFP4 only: block scales of w_o    [Hq d/128][D][4] */
  const uint8_t* mx_gu_s;    /* MXFP4 only: block scales of w_gu   [D/128][2F][4] */
  const uint8_t* mx_down_s;  /* MXFP4 only: block scales of w_down [F/128][D][4] */
  const float* awq_inv_o;    /* MXFP4 only: fp32 [Hq d] or NULL */
  const float* awq_inv_gu;   /* MXFP4 only: fp32 [D] or NULL */
} hr_layer;

/* KV cache of one layer: bf16 [n_slots * capacity, Hkv, d]; position p of the
 * sequence placed in slot s lives at row s * capacity + p.  Keys are stored
 * after q/k RMSNorm and RoPE (rotate-half order), values as projected. */
typedef struct {
  void* k;
  void* v;
  int32_t capacity;
  int32_t n_slots;
} hr_kv;

/* A packed varlen batch: the rows of sequence s are [cu_seqlens[s],
 * cu_seqlens[s+1]).  A single prompt of length P is n_seq = 1, cu = {0, P}.
 * Device arrays are read by the kernels; host mirrors (same contents) are
 * read by the validation.  used_keys / h_used_keys may be NULL when causal. */
typedef struct {
  int32_t n_seq;
  int32_t total_tokens;  /* T = cu_seqlens[n_seq] */
  int32_t max_seqlen;    /* >= every sequence length (HR_EBOUND otherwise) */
  const int32_t* cu_seqlens;   /* device [n_seq + 1] */
  const int32_t* start_pos;    /* device [n_seq]: position of the first row */
  const int32_t* cache_slot;   /* device [n_seq] */
  const int32_t* used_keys;    /* device [n_seq] (non-causal) */
  const int32_t* h_cu_seqlens; /* host mirrors */
  const int32_t* h_start_pos;
  const int32_t* h_cache_slot;
  const int32_t* h_used_keys;
} hr_batch;

/* Prepares one bf16 weight matrix of a layer for HR_F16_PACKED (once, at
 * load).  The four projection GEMMs of the chain ("Stabilize Higgs Audio
 * termination and prefill", Summary) stream these matrices; the layout serves
 * their tiles:
 *  w    bf16 [N, K] row-major (device), K a multiple of 32;
 *  out  device buffer of N * K * 2 bytes, not overlapping w: fp16 values in
 *       the slab-major layout out[K/32][N][32] (each 64-byte run is one row's
 *       32 consecutive K values, so the rows of a tile for one K slab are one
 *       contiguous run);
 *  gate_up 1 for w_gu ([gate; up], N = 2F, F a multiple of 32): packed row
 *       64 p + 32 u + r holds row u F + 32 p + r (32-row blocks alternate gate
 *       and up rows of the same activation columns); 0 for w_qkv, w_o, w_down.
 * The conversion is the one the HR_BF16 kernels make in registers (exact for
 * |w| in [2^-17, 65504], round to nearest even below 2^-17), so a layer of
 * packed weights computes the same products in the same order.  A weight
 * that does not fit fp16 (|w| >= 65520, inf, NaN) returns HR_EINVAL.  Unlike
 * the other entries this one synchronises `stream` (it reads that check back
 * from a one-word flag each GPU holds; packs that overlap on one GPU race on
 * it).  It allocates nothing. */
hr_status hr_pack_weight(const void* w, int32_t N, int32_t K, int32_t gate_up, void* out, hipStream_t stream);

/* Bytes of scratch the prefill calls need for `total_tokens` rows. */
size_t hr_workspace_bytes(const hr_dims* dims, hr_wtype wtype, int32_t total_tokens);

/* One decoder layer over a packed batch.
 *  h   fp32 [T, D], in/out: the residual stream (h <- layer(h)).
 *  kv  this layer's cache; rows of this batch's positions are written.
 *  ws  device scratch of at least hr_workspace_bytes(dims, layer->wtype, T). */
hr_status hr_prefill_layer(const hr_dims* dims, const hr_layer* layer, const hr_batch* batch,
                           float* h, const hr_kv* kv, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* The whole stack: h_0 = embed[ids] (or x_embeds when ids == NULL), layers
 * 0..L-1, then z = RMSNorm(h_L; final_norm_w).
 *  layers, kv   host arrays of L entries.
 *  embed        bf16 [vocab, D]; ids int32 [T] in [0, vocab) (not range-checked
 *               on the device: an out-of-range id is the caller's error).
 *  x_embeds     bf16 [T, D] input rows, used iff ids == NULL.
 *  h_out        fp32 [T, D]: receives h_L (the residual after the last layer).
 *  head_w       bf16 [K*V, D] or NULL; logits_out fp32 [n_seq, K, V] receives
 *               z(last row of each sequence) . head_w^T when both are given.
 * All layers must share one wtype. */
hr_status hr_prefill_stack(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch,
                           const int32_t* ids, const void* embed, int32_t vocab,
                           const void* x_embeds, const hr_kv* kv, const void* final_norm_w,
                           const void* head_w, int32_t n_codebooks, int32_t cb_vocab,
                           float* h_out, float* logits_out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* One delayed-codebook decode step for B streams (K codebooks of V ids).
 *  logits     [B, K, V], bf16 (logits_is_fp32 = 0) or fp32 (1).
 *  frame      int32 [B] in/out: decode step of each stream.
 *  eoc_seen   uint8 [B, K] in/out: codebook k has emitted EOC (sticky).
 *  done       uint8 [B] in/out: every codebook has emitted EOC.
 *  codes      int32 [B, K] out: the ids emitted this step.
 *  aligned    int32 [B, max_frames, K] or NULL: aligned frame f of codebook k
 *             is written at the step it is emitted (t = f + k), if f < max_frames.
 *  cb_embed   bf16 [K*V, D]; emb_out bf16 [B, D] = bf16(sum_k cb_embed[k*V+c_k])
 *             summed in fp32 in codebook order, rounded once (nearest-even).
 * Per stream: a done stream emits EOC everywhere and keeps its state.  Else with
 * t = frame: codebook k emits BOS while t < k, EOC if it already emitted EOC,
 * otherwise the lowest index of its row maximum; then frame = t+1 and
 * done = all codebooks have emitted EOC.
 * HR_EINVAL if bos_id or eoc_id is outside [0, V) or bos_id == eoc_id, or
 * D is not a multiple of 8; HR_EALIGN if logits, cb_embed or emb_out is not
 * 16-byte aligned. */
hr_status hr_codebook_step(int32_t B, int32_t K, int32_t V, int32_t bos_id, int32_t eoc_id,
                           int32_t logits_is_fp32, const void* logits, int32_t* frame,
                           uint8_t* eoc_seen, uint8_t* done, int32_t* codes, int32_t* aligned,
                           int32_t max_frames, const void* cb_embed, int32_t D, void* emb_out,
                           hipStream_t stream);

/* Per-stream sampling and termination policies for hr_codebook_step_policy.
 * Sampling (vLLM-Omni pull request 8226, Higgs Audio v3 streaming on Model
 * Runner V2, Purpose and Test Plan: temperature / top-k / top-p with per-request
 * seeded exponential noise).  All arrays are device memory of B entries, read
 * only; NULL means the default for every stream.
 *  temperature  fp32: > 0 samples from softmax(logits / T); <= 0 (or NULL) is
 *               the greedy argmax of hr_codebook_step.
 *  top_k        int32: keep the logits >= the k-th largest (ties at the k-th
 *               value stay); <= 0, >= V or NULL: off.
 *  top_p        fp32: order the survivors by logit (equal logits by lower id)
 *               and keep each while the softmax mass ahead of it is below p;
 *               >= 1 or NULL: off; <= 0 keeps the first only.
 *  seed         uint64: the stream's Philox4x64-10 key (seed, 0); row k at
 *               step t (= frame) draws counter block (t, k, v / 4, 0), word
 *               v % 4 for id v, u = (top 23 bits + 1/2) / 2^23; the winner is
 *               the kept id with the largest z - ln(-ln u) (lowest id on
 *               equality).  Required when temperature is given.
 * Termination (FlashRT pull request 141, Summary and Root cause: delayed EOC
 * for every codebook; a deterministic stop guard for repeated-code loops).  An
 * end frame e >= 0 forces codebook k to EOC at every step t >= e + k.
 *  eoc_cascade  1: when an open stream (e < 0) emits EOC in codebooks k1..kn
 *               at step t, e = t - max(k).
 *  repeat_limit 0: off; >= 2: an open stream counts consecutive steps whose K
 *               codes equal the previous step's (a new run counts 1) and sets
 *               e = t + 1 when the count reaches the limit.
 *  end_frame    int32 [B] in/out, -1 while open; required by either rule.
 *  last_codes   int32 [B, K] in/out (start at -1) and repeat_run int32 [B]
 *               in/out (start at 0): the guard's state, required by it. */
typedef struct {
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const uint64_t* seed;
  int32_t eoc_cascade;
  int32_t repeat_limit;
  int32_t* end_frame;
  int32_t* last_codes;
  int32_t* repeat_run;
} hr_step_policy;

/* hr_codebook_step with the policies above (policy NULL: all defaults, the
 * same codes as hr_codebook_step).  Per stream that is not done, with t = frame
 * and e = end_frame (-1 without one): codebook k emits BOS while t < k, EOC if
 * it already emitted EOC, EOC if e >= 0 and t >= e + k, else its row's choice
 * (greedy or sampled); then the guard and the cascade may set e (the smaller
 * of their candidates), frame = t + 1, done = every codebook has emitted EOC.
 * Arguments as for hr_codebook_step.  HR_EUNSUPPORTED if V > 2048; HR_EINVAL on
 * the checks of hr_codebook_step, temperature without seed, repeat_limit of 1
 * or below 0, or a missing state array; HR_EALIGN if seed is not 8-byte
 * aligned.  Calls that overlap on one stream state race. */
hr_status hr_codebook_step_policy(int32_t B, int32_t K, int32_t V, int32_t bos_id, int32_t eoc_id,
                                  int32_t logits_is_fp32, const void* logits, int32_t* frame,
                                  uint8_t* eoc_seen, uint8_t* done, int32_t* codes, int32_t* aligned,
                                  int32_t max_frames, const void* cb_embed, int32_t D, void* emb_out,
                                  const hr_step_policy* policy, hipStream_t stream);

/* One batched autoregressive decode step of B streams (the step that follows
 * the prefill, one new row per stream): the stack over x_embeds at each
 * stream's next position (its cache rows [0, start_pos] are attended
 * causally; long rows over few streams are split into key chunks), the audio
 * head on the new rows into logits_out, then the delayed-codebook step on
 * those logits, which writes this step's codes and the next step's input rows.
 *  batch       B sequences of one row each: cu_seqlens = {0, 1, ..., B},
 *              start_pos[b] = the position of stream b's new row (its cached
 *              length), cache_slot[b]; host mirrors as for the prefill.
 *  x_embeds    bf16 [B, D]: the new rows' input embeddings (for the step after
 *              a prefill: the codebook-embedding sum of its first codes).
 *  logits_out  fp32 [B, K, V]: the head's logits of this step (output).
 *  frame, eoc_seen, done, codes, aligned, max_frames, cb_embed: as in
 *              hr_codebook_step (D = dims->hidden).
 *  emb_out     bf16 [B, D]: the next step's x_embeds; may be the x_embeds buffer.
 *  ws          device scratch of at least hr_decode_workspace_bytes(dims, wtype, B).
 * HR_EUNSUPPORTED if dims->causal is 0; HR_EINVAL if a stream has other than one
 * row, head_w or logits_out is NULL, or on any check of hr_prefill_stack or
 * hr_codebook_step.  Nothing is launched when a check fails. */
size_t hr_decode_workspace_bytes(const hr_dims* dims, hr_wtype wtype, int32_t B);
hr_status hr_decode_step(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch,
                         const void* x_embeds, const hr_kv* kv, const void* final_norm_w,
                         const void* head_w, int32_t n_codebooks, int32_t cb_vocab, int32_t bos_id,
                         int32_t eoc_id, float* logits_out, int32_t* frame, uint8_t* eoc_seen,
                         uint8_t* done, int32_t* codes, int32_t* aligned, int32_t max_frames,
                         const void* cb_embed, void* emb_out, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* hr_decode_step without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, with their
 * scratch in a fixed device array of hr_decode_noalloc_scratch_bytes() (32 MiB)
 * that the library holds on each GPU it runs on until the process ends.  The
 * call allocates and frees nothing.  HR_EWORKSPACE when the step's scratch
 * (hr_decode_workspace_bytes) exceeds that size: up to 128 streams of the
 * 4B-class shape.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (two streams, two host threads) race and must be
 * serialised by the caller.  Other checks and errors as hr_decode_step. */
size_t hr_decode_noalloc_scratch_bytes(void);
hr_status hr_decode_step_noalloc(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch,
                                 const void* x_embeds, const hr_kv* kv, const void* final_norm_w,
                                 const void* head_w, int32_t n_codebooks, int32_t cb_vocab, int32_t bos_id,
                                 int32_t eoc_id, float* logits_out, int32_t* frame, uint8_t* eoc_seen,
                                 uint8_t* done, int32_t* codes, int32_t* aligned, int32_t max_frames,
                                 const void* cb_embed, void* emb_out, hipStream_t stream);

const char* hr_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HR_H */
