/*
 * hr_ops.h -- the individual steps of the prefill chain declared in hr.h, each
 * exposed on its own so that a caller (or a test) can run and check one step.
 * hr_prefill_layer / hr_prefill_stack run exactly these kernels in this order.
 * Conventions (ownership, alignment, errors, streams) are those of hr.h.
 *
 * Sources, by page title and section: flashrt-structures 0.2.0
 * prefill_tower/fp8_chain.py (module docstring; `run`; `_build_rope`;
 * `_prefill_mask_facts`; the quantiser table of `_quantize`), and
 * "Stabilize Higgs Audio termination and prefill", Summary.
 */
#ifndef HR_OPS_H
#define HR_OPS_H

#include "hr.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Embedding lookup + input RMSNorm (steps A0, A1).
 * h_out[t] = embed[ids[t]] widened to fp32 (x_embeds[t] when ids == NULL);
 * x_out[t] = h[t] * (mean(h[t]^2) + eps)^-1/2 * norm_w, stored fp16
 * (x_type == HR_F16, the input of the bf16-weight band's GEMMs) or as
 * e4m3(x / x_scale) (x_type == HR_FP8_E4M3).  D a multiple of 8. */
hr_status hr_embed_rmsnorm(const int32_t* ids, const void* embed, int32_t vocab,
                           const void* x_embeds, int32_t T, int32_t D, const void* norm_w,
                           float eps, float* h_out, void* x_out, hr_wtype x_type, float x_scale,
                           hipStream_t stream);

/* RMSNorm of the fp32 residual (steps A6, A9): x_out[t] = RMS(h[t]) * norm_w,
 * fp16 (HR_F16) or e4m3(x / x_scale) (HR_FP8_E4M3).  (The residual add itself
 * is fused into the epilogue of the O and down projections, HR_EPI_RESIDUAL.) */
hr_status hr_rmsnorm(const float* h, int32_t T, int32_t D, const void* norm_w, float eps,
                     void* x_out, hr_wtype x_type, float x_scale, hipStream_t stream);

typedef enum {
  HR_EPI_F32 = 0,       /* out fp32 [M, N] = x W^T  (the merged QKV rows)        */
  HR_EPI_RESIDUAL = 1,  /* out fp32 [M, N] += x W^T  (residual add)              */
  HR_EPI_SWIGLU = 2,    /* N = 2F (gate rows, then up rows); out [M, F] =
                           silu(g) * u, fp16, or e4m3(./out_scale) in FP8 mode  */
  HR_EPI_RANGE_MIN_ = INT32_MIN, HR_EPI_RANGE_MAX_ = INT32_MAX   /* range markers, as for hr_wtype */
} hr_epilogue;

/* Projection (steps A2, A5, A7, A8): x [M, K] times W [N, K]^T, fp32
 * accumulation.
 * HR_EPI_RESIDUAL may split K over workgroups to fill the GPU; the splits'
 * fp32 partials then go to ws (hr_linear_workspace_bytes: 0 when no split is
 * taken) and are added to out in split order, h + (p0 + p1 + ...): the
 * result does not depend on the order in which workgroups finish, and equals
 * bit for bit what the layer entries compute (there the add is fused with the
 * next RMSNorm, hr_residual_rmsnorm).  HR_EWORKSPACE if ws is too small.
 *  wtype HR_BF16:     x fp16, w bf16 (each weight enters the fp16 MFMA
 *                     converted exactly: bf16 values of magnitude 2^-17 to
 *                     2^16 are fp16 values; smaller ones round to a multiple
 *                     of 2^-24); w_scale ignored.
 *  wtype HR_FP8_E4M3: x and w e4m3; the product is scaled by
 *                     x_scale * w_scale[n].
 *  wtype HR_F16_PACKED: x fp16, w written by hr_pack_weight (gate_up = 1 for
 *                     SWIGLU, N then a multiple of 64); bit for bit the
 *                     HR_BF16 result of the unpacked weights; w_scale ignored.
 * K a multiple of 64, N a multiple of 16 (32 for SWIGLU). */
size_t hr_linear_workspace_bytes(hr_wtype wtype, int32_t M, int32_t N, int32_t K, hr_epilogue epi);
hr_status hr_linear(const void* x, const void* w, const float* w_scale, float x_scale,
                    hr_wtype wtype, int32_t M, int32_t N, int32_t K, hr_epilogue epi, void* out,
                    float out_scale, void* ws, size_t ws_bytes, hipStream_t stream);

/* Fused residual add + RMSNorm (steps A6, A9; the fused residual-add +
 * RMSNorm (+ quantise) of flashrt-structures prefill_tower/fp8_chain.py, `run`):
 * h[t] += p[0][t] + ... + p[n-1][t] with p[k] = partials + k*T*D (the split-K
 * partials of a residual projection, summed in that order, then added to h;
 * n_partials = 0: no add), then x_out[t] = RMS(h[t]) * norm_w as fp16
 * (HR_F16) or e4m3(x / x_scale); x_out NULL: the add alone.  h fp32 [T, D],
 * D a multiple of 8 and <= 8192. */
hr_status hr_residual_rmsnorm(float* h, const float* partials, int32_t n_partials, int32_t T, int32_t D,
                              const void* norm_w, float eps, void* x_out, hr_wtype x_type, float x_scale,
                              hipStream_t stream);

/* Per-head q/k RMSNorm + rotate-half RoPE + KV-cache write (step A3).
 * qkv fp32 [T, (Hq+2Hkv)d] -> q_out fp16 [T, Hq, d] (normed, rotated);
 * cache rows slot*capacity + start_pos + i receive k (normed, rotated) and v,
 * each rounded once to bf16.
 * RoPE angle of pair (m, m + d/2) at position p: p * theta^(-2m/d).
 * Non-causal batches skip the cache write of pad rows i >= used_keys[s]. */
hr_status hr_qknorm_rope_kv(const hr_dims* dims, const hr_batch* batch, const void* qkv,
                            const void* q_norm_w, const void* k_norm_w, void* q_out,
                            const hr_kv* kv, hipStream_t stream);

/* Steps A3 and A4 in one launch for short prompts: the q/k norm + RoPE + KV
 * write of hr_qknorm_rope_kv (the cache receives the same values) followed by
 * the attention of hr_attention, out fp16 (HR_F16) or e4m3(o / out_scale)
 * [T, Hq*d],
 * without writing q anywhere.  Every sequence must start at position 0 and
 * hold at most 32 rows (HR_EUNSUPPORTED otherwise): its keys are then its own
 * rows.  The layer entries take this path by themselves for such batches. */
hr_status hr_qknorm_rope_attention(const hr_dims* dims, const hr_batch* batch, const void* qkv,
                                   const void* q_norm_w, const void* k_norm_w, const hr_kv* kv, void* out,
                                   hr_wtype out_type, float out_scale, hipStream_t stream);

/* GQA attention over the cache (step A4): q fp16 [T, Hq, d], out [T, Hq*d]
 * with o_h = softmax(q_h K_g^T / sqrt(d)) V_g, g = h / (Hq/Hkv), over the
 * causal window or the used keys (dims->causal).  Scores and P V run as fp16
 * MFMAs with fp32 accumulation (the bf16 cache rows convert exactly); out fp16
 * (HR_F16) or e4m3(o / out_scale) (HR_FP8_E4M3). */
hr_status hr_attention(const hr_dims* dims, const hr_batch* batch, const void* q, const hr_kv* kv,
                       void* out, hr_wtype out_type, float out_scale, hipStream_t stream);

/* The attention of hr_attention (step A4) for a batch whose keys are all its
 * own rows -- every sequence starts at position 0 (HR_EUNSUPPORTED otherwise)
 * -- read from fp16 copies instead of the cache: k16 and v16 [Tp][Hkv][d],
 * row t the key / value row of batch row t; rows past the batch's T rows
 * finite (zero); Tp a multiple of 32, at least T rounded up to 32 (HR_EINVAL).
 * Every sequence must start at a batch row that is a multiple of 8
 * (HR_EUNSUPPORTED).  These are the copies the layer entries' fused QKV +
 * step A3 launch writes for causal batches of 385-1024 rows (the cache's bf16
 * values widened to fp16, exact), and the layer entries take this path by
 * themselves there.  The
 * tiles go HBM -> LDS without conversion; a workgroup takes one query head and
 * the 32-row query blocks p and nb-1-p of a sequence, 4 streams of 32-key
 * tiles each feeding a wave of both blocks, the streams' partial softmaxes
 * merged in a fixed order.  q, out and the tolerances as
 * in hr_attention; all pointers device memory, 16-byte aligned (HR_EALIGN);
 * nothing is allocated. */
hr_status hr_attention_f16(const hr_dims* dims, const hr_batch* batch, const void* q, const void* k16,
                           const void* v16, int32_t Tp, void* out, hr_wtype out_type, float out_scale,
                           hipStream_t stream);

/* The same attention with each query block's keys split into chunks that run
 * in separate workgroups (more parallel work for a few long rows), followed by
 * a merge: chunk c keeps its running max m_c (base 2), sum l_c and unnormalised
 * o_c in fp32, and o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c with
 * M = max_c m_c, the standard combination of partial softmaxes.  A query block
 * of n 64-key tiles takes max(chunk_tiles, ceil(n / n_slots)) tiles per chunk;
 * blocks of at most chunk_tiles tiles are not split.  chunk_tiles >= 1,
 * 1 <= n_slots <= 64.  ws: device scratch of at least
 * hr_attention_chunked_workspace_bytes(dims, T, n_slots) bytes, 256-byte
 * aligned (HR_EWORKSPACE / HR_EALIGN otherwise).  Worth it for rows much
 * longer than the batch (a short continuation of a long cached prefix): a
 * prefill from position 0 already has one query block per 32 rows. */
size_t hr_attention_chunked_workspace_bytes(const hr_dims* dims, int32_t total_tokens, int32_t n_slots);
hr_status hr_attention_chunked(const hr_dims* dims, const hr_batch* batch, const void* q, const hr_kv* kv,
                               void* out, hr_wtype out_type, float out_scale, int32_t chunk_tiles,
                               int32_t n_slots, void* ws, size_t ws_bytes, hipStream_t stream);

/* Final RMSNorm + audio-head projection of each sequence's last row
 * (steps A9 final, A10): z = RMS(h[last_s]; final_norm_w) in fp32, then
 * logits[s, k, v] = z . head_w[k*V + v] in fp32 (z is split into two bf16
 * terms so the product keeps fp32 accuracy).  ws >= hr_head_workspace_bytes. */
size_t hr_head_workspace_bytes(int32_t n_seq, int32_t D);
hr_status hr_head_logits(const float* h, const hr_batch* batch, int32_t D, const void* final_norm_w,
                         float eps, const void* head_w, int32_t n_codebooks, int32_t cb_vocab,
                         float* logits_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* FP8 weight packing: scale[n] = max_k |w[n, k]| / 448 (1 if the row is zero),
 * w8[n, k] = e4m3(w[n, k] / scale[n]) with fp32 division, nearest-even,
 * saturating at 448.  w bf16 [N, K]. */
hr_status hr_quantize_weight_e4m3(const void* w, int32_t N, int32_t K, uint8_t* w8, float* scale,
                                  hipStream_t stream);

/* ---- MXFP4 band of the O and FFN projections (NEXT-4) -------------------
 * flashrt-structures 0.2.0, prefill_tower/fp8_chain.py: the FP4 band table (the
 * FFN pair and the attention output projection in 4-bit with dynamic block
 * scales, QKV unchanged), _awq_scale (per-input-channel pre-scale s; the GEMM
 * columns carry s, the tensor feeding the GEMM carries 1/s) and
 * _interleave_gu_rows (the down projection's 1/s folded into the up rows).  On
 * gfx950 the format is OCP MX FP4: E2M1 values (0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 * negatives; nearest, ties to the even code, saturating at 6), one E8M0 scale
 * 2^e per 32 consecutive values along K, e = floor(log2 max|v|) - 2 clamped to
 * [-127, 127] (byte e + 127; an all-zero block gets byte 0).
 * Layouts: codes u8 [rows, K/2], element 2i in the low nibble of byte i;
 * scales u8 in the slab-interleaved layout [K/128][ld][4] (block kb of row r at
 * ((kb/4) * ld + r) * 4 + kb % 4), ld >= rows.  K must be a multiple of 128;
 * codes, scales and the scale vectors 16-byte aligned. */

/* Quantise rows: v = x[r, k] * col_scale[k] * row_scale[r] (each product one
 * binary32 rounding, in that order; a NULL vector is 1), then MX blocks.
 * x [M, K] in the format x_format: 0 bf16 (weights), 1 fp32, 2 fp16 (the
 * attention output of the MXFP4 band).  Weights: col_scale = AWQ s of the input
 * channels, row_scale = 1/s of the down projection on the up rows.
 * Activations: col_scale = 1/s.  HR_EINVAL on sizes or ld_scales < M. */
hr_status hr_quantize_mxfp4(const void* x, int32_t x_format, int32_t M, int32_t K, const float* col_scale,
                            const float* row_scale, uint8_t* codes, uint8_t* scales, int32_t ld_scales,
                            hipStream_t stream);

/* x = RMS(h; norm_w) * col_scale straight to MXFP4 (the gate/up input with its
 * 1/s).  h fp32 [T, D], D a multiple of 128 and <= 8192. */
hr_status hr_rmsnorm_mxfp4(const float* h, int32_t T, int32_t D, const void* norm_w, float eps,
                           const float* col_scale, uint8_t* codes, uint8_t* scales, int32_t ld_scales,
                           hipStream_t stream);

/* MXFP4 GEMM y = x w^T with fp32 accumulation of the scaled E2M1 products.
 *  ws / ws_bytes: the split-K partials of HR_EPI_RESIDUAL, as for hr_linear
 *  (hr_linear_workspace_bytes(HR_MXFP4, ...)).
 *  x codes [M, K/2] with scales (ld_x_scales >= M rounded up to 256: the
 *  256-row tiles read whole scale rows; rows >= M are ignored), w codes
 *  [N, K/2] with scales (ld N).
 *  HR_EPI_RESIDUAL: out fp32 [M, N] += y (N a multiple of 256).
 *  HR_EPI_SWIGLU: N = 2F, w rows [gate; up]; act = silu(gate) * up goes out as
 *  MXFP4: codes [M, F/2] into out, scales into out_scales with ld_out_scales
 *  (>= M rounded up to 256, so the result can feed this call as x); F a
 *  multiple of 128. */
hr_status hr_linear_mxfp4(const uint8_t* x, const uint8_t* x_scales, int32_t ld_x_scales, const uint8_t* w,
                          const uint8_t* w_scales, int32_t M, int32_t N, int32_t K, hr_epilogue epi, void* out,
                          uint8_t* out_scales, int32_t ld_out_scales, void* ws, size_t ws_bytes,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HR_OPS_H */
