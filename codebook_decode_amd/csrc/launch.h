// Internal launchers of libhr's kernels (host side).  Shapes are validated by
// api.cpp before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hr_ops.h"

namespace hr {

constexpr int HR_EPI_HEAD = 3;        // internal: fp32 logits from hi/lo bf16 rows
constexpr int HR_EPI_QKV_ROPE = 5;    // internal: merged QKV rows -> q/k norm + RoPE + KV write


void launch_codebook_step(int B, int K, int V, int bos, int eoc, bool f32, const void* logits,
                          int32_t* frame, uint8_t* eoc_seen, uint8_t* done, int32_t* codes,
                          int32_t* aligned, int max_frames, const void* cb_embed, int D,
                          void* emb_out, hipStream_t st);

// per-stream sampling and termination policies (fields as hr_step_policy)
struct StepPolicy {
  const float* temperature = nullptr;
  const int32_t* top_k = nullptr;
  const float* top_p = nullptr;
  const uint64_t* seed = nullptr;
  int eoc_cascade = 0;
  int repeat_limit = 0;
  int32_t* end_frame = nullptr;
  int32_t* last_codes = nullptr;
  int32_t* repeat_run = nullptr;
};
void launch_codebook_policy(int B, int K, int V, int bos, int eoc, bool f32, const void* logits,
                            int32_t* frame, uint8_t* eoc_seen, uint8_t* done, int32_t* codes,
                            int32_t* aligned, int max_frames, const void* cb_embed, int D,
                            void* emb_out, const StepPolicy& pol, hipStream_t st);

void launch_embed_rmsnorm(const int32_t* ids, const void* embed, const void* x_embeds, int T, int D,
                          const void* w, float eps, float* h_out, void* x_out, bool fp8,
                          float inv_scale, hipStream_t st);
void launch_rmsnorm(const float* h, int T, int D, const void* w, float eps, void* x_out, bool fp8,
                    float inv_scale, hipStream_t st);
void launch_final_split(const float* h, const int32_t* cu, int seq0, int n, int D, const void* w,
                        float eps, int n_rows, void* zsplit, hipStream_t st);
void launch_quant_weight(const void* w, int N, int K, uint8_t* w8, float* scale, hipStream_t st);
// MXFP4: codes [M, K/2] (two per byte, element 2i low), scales in the
// slab-interleaved layout [K/128][ld_s][4] (ld_s >= M)
// fmt: 0 bf16, 1 fp32, 2 fp16 rows
void launch_quant_mx(const void* x, int fmt, int M, int K, const float* col, const float* row_scale,
                     uint8_t* codes, uint8_t* scales, int ld_s, hipStream_t st);
void launch_rmsnorm_mx(const float* h, int T, int D, const void* w, const float* col, float eps,
                       uint8_t* codes, uint8_t* scales, int ld_s, hipStream_t st);

void launch_qknorm_rope_kv(const void* qkv, int T, int Hq, int Hkv, int d, float theta, float eps,
                           const int32_t* cu, const int32_t* start_pos, const int32_t* cache_slot,
                           const int32_t* used_keys, int n_seq, bool causal, const void* qw,
                           const void* kw, void* q_out, void* kc, void* vc, int capacity,
                           hipStream_t st);

// Short prompts from position 0 (every sequence at most kSmallRows rows):
// q/k norm + RoPE + KV write and the attention in one launch, grid (Hq, n_seq)
constexpr int kSmallRows = 32;
// tab: the batch's RoPE angle table (launch_rope_table), or null: the
// workgroups compute the angles of their rows themselves (the same bits)
void launch_rope_attn_small(const void* qkv, int n_seq, int max_len, int Hq, int Hkv, int d, float theta, float eps,
                            const int32_t* cu, const int32_t* cache_slot, const int32_t* used_keys, bool causal,
                            const void* qw, const void* kw, void* kc, void* vc, int capacity, void* out, bool fp8,
                            float out_inv, hipStream_t st, const float* tab = nullptr);

// Key-chunk split of the attention (more workgroups for long rows): query
// blocks with more than chunk_tiles 64-key tiles write fp32 partials per chunk
// (n_slots chunk slots at most) and a merge kernel combines them.
struct AttnSplit {
  bool decode = false;      // one row per sequence: decode_attention_kernel (+ merge when chunked)
  int groups = 1;           // wave groups interleaving the key tiles of a block (1 or 2)
  int head_split = 1;       // workgroups sharing a KV head's query heads (1 or 2)
  int chunk_tiles = 0;      // 0: no split
  int n_slots = 1;
  float* part_o = nullptr;  // [n_slots, T, Hq, d]
  float* part_ml = nullptr; // [n_slots, T, Hq, 2]: running max (log2 units), sum
  int T = 0;
};
int attention_qpw(int Hq, int Hkv);
void launch_attention(const void* q, const void* kc, const void* vc, const int32_t* cu,
                      const int32_t* sp, const int32_t* slot, const int32_t* used, int n_seq,
                      int max_len, int Hq, int Hkv, int d, int cap, bool causal, void* out, bool fp8,
                      float out_inv, hipStream_t st, const AttnSplit* split = nullptr);

// Attention of a batch whose keys are all its own rows (every sequence starts
// at position 0) from the fp16 copies the QKV + step A3 launch wrote (QkvRope
// k16 / v16, Tp rows): grid (query-block pairs, Hq, n_seq), d 64 or 128.
void launch_attention_f16(const void* q, const void* k16, const void* v16, int Tp, const int32_t* cu,
                          const int32_t* used, int n_seq, int max_len, int Hq, int Hkv, int d, bool causal,
                          void* out, bool fp8, float out_inv, hipStream_t st);

// Decode steps (one row per sequence, causal): step A3 (q/k norm, RoPE, the new
// row's K/V write) inside the decode attention launch; qkv = the merged QKV rows.
void launch_decode_rope_attention(const void* qkv, const void* qw, const void* kw, float theta, float eps,
                                  void* kc, void* vc, const int32_t* cu, const int32_t* sp, const int32_t* slot,
                                  int n_seq, int Hq, int Hkv, int d, int cap, void* out, bool fp8, float out_inv,
                                  const AttnSplit& cfg, hipStream_t st);

// Projections.  Return the split-K factor ks of the launch (1 unless the
// epilogue is HR_EPI_RESIDUAL).  RESIDUAL with ks > 1 writes ks fp32 partials
// [ks][M][N] to `part` instead of touching `out`; the caller reduces them
// (launch_residual_norm).  go == false: plan only (return ks, launch nothing).
// packed: w is fp16 in the slab-major layout of launch_pack_weight (fp8 false)
int launch_linear(const void* x, const void* w, const float* w_scale, float x_scale, bool fp8, bool packed,
                  int M, int N, int K, int epi, void* out, float out_scale, float* part, bool go,
                  hipStream_t st);
// Merged QKV projection with step A3 in its epilogue: the fp32 rows of each
// 128-column tile (whole heads) are normed (q / k, own weights), rotated and
// written as the separate step writes them (q fp16 [T, Hq, d], K / V rows bf16
// into the cache), with the angles from launch_rope_table's table.  Takes
// 384 < M <= 1024 and d in {64, 128}; returns false (nothing launched)
// otherwise.
struct QkvRope {
  void* q_out;
  void* kc;
  void* vc;
  const int32_t* cu;
  const int32_t* start_pos;
  const int32_t* cache_slot;
  const int32_t* used_keys;
  int n_seq, causal, capacity, Hq, Hkv, d;
  const void* qw;
  const void* kw;
  float eps;
  const float* rope;   // [T][d]: cos of pairs m < d/2, then their sin
  // optional fp16 copies of this batch's keys and values for attention_f16
  // (null: none): k16 and v16 [Tp][Hkv][d], the cache's rows widened to fp16
  // (exact); rows T..Tp-1 zero (Tp = T rounded up to 32)
  void* k16;
  void* v16;
  int Tp;
};
bool qkv_rope_fits(int M, int d);
bool launch_qkv_rope(const void* x, const void* w, const float* w_scale, float x_scale, bool fp8, bool packed,
                     int M, int K, const QkvRope& qr, hipStream_t st);
// the RoPE angle table of a batch: tab[t][m] = cos, tab[t][d/2 + m] = sin of
// position(t) * theta^(-2m/d) (the same arithmetic as the q/k norm kernels)
void launch_rope_table(const int32_t* cu, const int32_t* start_pos, int n_seq, int T, int d, float theta,
                       float* tab, hipStream_t st);
// bf16 W [N, K] -> packed fp16 (slab-major [K/32][N][32], gate_up: 32-row
// gate / up blocks); synchronous; 0 ok, 1 a non-finite fp16 value, -1 HIP error
int launch_pack_weight(const void* w, int N, int K, bool gate_up, void* out, hipStream_t st);
int launch_linear_mx(const uint8_t* x, const uint8_t* x_scales, int lda, const uint8_t* w,
                     const uint8_t* w_scales, int M, int N, int K, int epi, void* out, uint8_t* out_scales,
                     int ldo, float* part, bool go, hipStream_t st);

// h[t] += sum over kz = 0..ks-1 of part[kz][t] (in that order; ks = 0: no
// add), then, when out_mode != kNormNone, x = RMS(h[t]) * w (* col for MX)
// in the out_mode format.  One workgroup per row.
enum NormOut { kNormNone = 0, kNormF16 = 1, kNormE4M3 = 2, kNormMX = 3 };
// the residual add alone over a flat array of n elements (n % 8 == 0), in the
// order and arithmetic of launch_residual_norm
void launch_residual_sum(float* h, const float* part, int ks, size_t n, hipStream_t st);
void launch_residual_norm(float* h, const float* part, int ks, int T, int D, const void* w, float eps,
                          int out_mode, void* x_out, float inv_scale, const float* col, uint8_t* mx_scales,
                          int mx_ld, hipStream_t st);
void launch_head_gemm(const void* zsplit, int n, const void* w, int N, int D, float* out,
                      hipStream_t st);

}  // namespace hr
