// libhr C ABI: host-side validation and the launch sequence of the prefill
// chain and the delayed-codebook step.  Every check runs before the first
// launch, so a failing call enqueues nothing.  No device memory is allocated,
// freed or read here; all work goes to the caller's stream.
//
// Launch order of one layer (flashrt-structures prefill_tower/fp8_chain.py,
// `run`, with the residual kept in fp32 and added inside the O / down GEMM
// epilogues):
//   rmsnorm(in) -> QKV GEMM -> q/k norm + RoPE + KV write -> attention ->
//   O GEMM (h +=) -> rmsnorm(post) -> gate/up GEMM + SwiGLU -> down GEMM (h +=)
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "hr.h"
#include "hr_ops.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

hr_status fail(hr_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HR_TRY(expr)                  \
  do {                                \
    hr_status _s = (expr);            \
    if (_s != HR_OK) return _s;       \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hr_status need(const void* p, const char* name) {
  if (p == nullptr) return fail(HR_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(HR_EALIGN, "%s is not 16-byte aligned", name);
  return HR_OK;
}

hr_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HR_EHIP, "%s: %s", what, hipGetErrorString(e));
  return HR_OK;
}

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

hr_status check_dims(const hr_dims* d) {
  if (!d) return fail(HR_EINVAL, "dims is NULL");
  if (d->hidden <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 || d->ffn <= 0)
    return fail(HR_EINVAL, "non-positive dimension");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(HR_EUNSUPPORTED, "head_dim %d not in {64, 128}", d->head_dim);
  if (d->n_q_heads % d->n_kv_heads != 0) return fail(HR_EUNSUPPORTED, "n_q_heads %% n_kv_heads != 0");
  const int group = d->n_q_heads / d->n_kv_heads;
  if (group != 1 && group != 2 && group != 4)
    return fail(HR_EUNSUPPORTED, "query heads per kv head %d not in {1, 2, 4}", group);
  if (d->hidden % 64 || d->ffn % 64) return fail(HR_EUNSUPPORTED, "hidden and ffn must be multiples of 64");
  if (d->hidden > 8192) return fail(HR_EUNSUPPORTED, "hidden %d > 8192", d->hidden);
  // the tiled GEMM addresses each operand with 32-bit byte offsets
  if (uint64_t(2) * d->ffn * d->hidden * 2 >= (uint64_t(1) << 32))
    return fail(HR_EUNSUPPORTED, "gate/up weight of %d x %d exceeds 4 GB", 2 * d->ffn, d->hidden);
  if (!(d->rope_theta > 0.f) || !(d->rms_eps >= 0.f) || !std::isfinite(d->rope_theta))
    return fail(HR_EINVAL, "rope_theta must be > 0 and rms_eps >= 0");
  return HR_OK;
}

hr_status check_kv(const hr_dims* d, const hr_kv* kv, const char* name) {
  if (!kv) return fail(HR_EINVAL, "%s is NULL", name);
  HR_TRY(need(kv->k, "kv.k"));
  HR_TRY(need(kv->v, "kv.v"));
  if (kv->capacity <= 0 || kv->n_slots <= 0) return fail(HR_EINVAL, "%s: capacity and n_slots must be > 0", name);
  (void)d;
  return HR_OK;
}

hr_status check_batch(const hr_dims* d, const hr_batch* b, const hr_kv* kv) {
  if (!b) return fail(HR_EINVAL, "batch is NULL");
  if (b->n_seq <= 0) return fail(HR_EINVAL, "n_seq must be > 0");
  if (!b->h_cu_seqlens || !b->h_start_pos || !b->h_cache_slot)
    return fail(HR_EINVAL, "host mirrors of cu_seqlens / start_pos / cache_slot are required");
  if (!b->cu_seqlens || !b->start_pos || !b->cache_slot)
    return fail(HR_EINVAL, "device cu_seqlens / start_pos / cache_slot are required");
  if (!d->causal && (!b->used_keys || !b->h_used_keys))
    return fail(HR_EINVAL, "non-causal batches need used_keys (device and host)");
  const int32_t* cu = b->h_cu_seqlens;
  if (cu[0] != 0) return fail(HR_EINVAL, "cu_seqlens[0] = %d, expected 0", cu[0]);
  for (int s = 0; s < b->n_seq; ++s) {
    const int len = cu[s + 1] - cu[s];
    if (len < 0) return fail(HR_EINVAL, "cu_seqlens not monotone at %d", s);
    if (len > b->max_seqlen)
      return fail(HR_EBOUND, "sequence %d has %d rows > max_seqlen %d", s, len, b->max_seqlen);
    const int sp = b->h_start_pos[s], slot = b->h_cache_slot[s];
    if (sp < 0) return fail(HR_EINVAL, "start_pos[%d] = %d < 0", s, sp);
    if (slot < 0 || slot >= kv->n_slots)
      return fail(HR_ECAPACITY, "cache_slot[%d] = %d outside [0, %d)", s, slot, kv->n_slots);
    if (int64_t(sp) + len > kv->capacity)
      return fail(HR_ECAPACITY, "sequence %d: start_pos %d + %d rows > capacity %d", s, sp, len, kv->capacity);
    if (!d->causal) {
      const int u = b->h_used_keys[s];
      if (sp != 0) return fail(HR_EUNSUPPORTED, "non-causal sequences must start at position 0");
      if (len > 0 && u < 1) return fail(HR_EINVAL, "used_keys[%d] = %d < 1", s, u);
      if (u > len) return fail(HR_EBOUND, "used_keys[%d] = %d > %d rows", s, u, len);
    }
  }
  if (cu[b->n_seq] != b->total_tokens)
    return fail(HR_EINVAL, "cu_seqlens[n_seq] = %d != total_tokens %d", cu[b->n_seq], b->total_tokens);
  {
    const int64_t widest = d->ffn > d->hidden ? d->ffn : d->hidden;
    const int64_t attn = int64_t(d->n_q_heads) * d->head_dim;
    if (int64_t(b->total_tokens) * (widest > attn ? widest : attn) * 2 >= (int64_t(1) << 32))
      return fail(HR_EUNSUPPORTED, "%d tokens: an activation matrix exceeds 4 GB", b->total_tokens);
  }
  return HR_OK;
}

hr_status check_layer(const hr_dims* d, const hr_layer* L, int idx) {
  if (!L) return fail(HR_EINVAL, "layer %d is NULL", idx);
  if (L->wtype != HR_BF16 && L->wtype != HR_FP8_E4M3 && L->wtype != HR_MXFP4 && L->wtype != HR_F16_PACKED)
    return fail(HR_EINVAL, "layer %d: bad wtype", idx);
  const void* ptrs[] = {L->in_norm_w, L->post_norm_w, L->q_norm_w, L->k_norm_w,
                        L->w_qkv,     L->w_o,         L->w_gu,     L->w_down};
  const char* names[] = {"in_norm_w", "post_norm_w", "q_norm_w", "k_norm_w", "w_qkv", "w_o", "w_gu", "w_down"};
  for (int i = 0; i < 8; ++i) {
    if (!ptrs[i]) return fail(HR_EINVAL, "layer %d: %s is NULL", idx, names[i]);
    if (!aligned16(ptrs[i])) return fail(HR_EALIGN, "layer %d: %s is not 16-byte aligned", idx, names[i]);
  }
  if (L->wtype == HR_FP8_E4M3) {
    if (!L->ws_qkv || !L->ws_o || !L->ws_gu || !L->ws_down)
      return fail(HR_EINVAL, "layer %d: FP8 weight scales missing", idx);
    const float a[] = {L->as_qkv, L->as_o, L->as_gu, L->as_down};
    for (float v : a)
      if (!(v > 0.f) || !std::isfinite(v))
        return fail(HR_EINVAL, "layer %d: FP8 activation scales must be finite and > 0", idx);
    // e4m3 GEMMs step K in slabs of up to 128 values
    if (d->hidden % 128 || d->ffn % 128 || (d->n_q_heads * d->head_dim) % 128)
      return fail(HR_EUNSUPPORTED, "layer %d: FP8 needs D, F and Hq d to be multiples of 128", idx);
  }
  if (L->wtype == HR_MXFP4) {
    const uint8_t* sc[] = {L->mx_o_s, L->mx_gu_s, L->mx_down_s};
    for (const uint8_t* p : sc) {
      if (!p) return fail(HR_EINVAL, "layer %d: MXFP4 block scales missing", idx);
      if (!aligned16(p)) return fail(HR_EALIGN, "layer %d: MXFP4 block scales not 16-byte aligned", idx);
    }
    if ((L->awq_inv_o && !aligned16(L->awq_inv_o)) || (L->awq_inv_gu && !aligned16(L->awq_inv_gu)))
      return fail(HR_EALIGN, "layer %d: AWQ vectors not 16-byte aligned", idx);
    const int A = d->n_q_heads * d->head_dim;
    if (d->hidden % 256 || A % 128 || d->ffn % 128)
      return fail(HR_EUNSUPPORTED, "layer %d: MXFP4 needs D %% 256, Hq d %% 128, F %% 128 == 0", idx);
  }
  return HR_OK;
}

struct Ws {
  uint8_t *x, *qkv, *q, *attn, *act, *head;
  float* rope;               // RoPE angle table [T][d] of the QKV epilogue (cos, then sin)
  float* part;               // split-K partials of the O / down projections [ks][T][D] (null: none needed)
  float *part_o, *part_ml;   // key-chunk partials of the split attention (null: no split)
  uint8_t *mx_s1, *mx_s2;    // MXFP4 block scales: O / gate-up input, down input (ld mx_ld)
  int mx_ld;                 // rows of the scale layouts: T rounded up to the 256-row tile
  uint8_t *k16, *v16;        // fp16 copies of the batch's K and V rows [Tp][Hkv][d] (null: none)
  int Tp;                    // their rows: T rounded up to 32
};

// Batches of up to kAttnSplitT rows may split long attention rows into key
// chunks (decode steps and short continuations of long cached prefixes).
constexpr int kAttnSplitT = 256;
constexpr int kAttnSlots = 4;      // key chunks per query block at most
constexpr int kDecodeSlotRows = 256;        // partial rows (chunks x tokens) reserved for decode steps at least
constexpr int kDecodeMaxSlots = 8;          // key chunks of a decode row at most
constexpr long long kDecodeGrid = 512;      // workgroups a decode step's chunking aims at
constexpr int kAttnMinChunk = 8;   // 64-key tiles per chunk of the longest row at least
constexpr int kAttnChunk = 4;      // 64-key tiles per chunk of shorter rows at least
constexpr long long kAttnSplitGrid = 512;   // workgroups of a split grid at most

// rows (key chunk x token) of the attention partials in the workspace
size_t part_rows(size_t t) {
  const size_t r = size_t(kAttnSlots) * t;
  return r > size_t(kDecodeSlotRows) ? r : size_t(kDecodeSlotRows);
}

// Largest split-K factor the residual projections (O: K = Hq d, down: K = F;
// N = D, M = T rows) take in any weight format: the partial buffer holds that
// many [T, D] fp32 slices.
int residual_ks(const hr_dims* d, int32_t T) {
  if (T <= 0) return 1;
  const int D = d->hidden, A = d->n_q_heads * d->head_dim, F = d->ffn;
  int ks = 1;
  for (int K : {A, F}) {
    // bf16, e4m3, packed fp16 (each format plans its own tiles)
    for (int f = 0; f < 3; ++f) {
      const bool fp8 = f == 1, pk = f == 2;
      if (fp8 && K % 128) continue;
      const int k = hr::launch_linear(nullptr, nullptr, nullptr, 1.f, fp8, pk, T, D, K, HR_EPI_RESIDUAL, nullptr, 0.f,
                                      nullptr, false, nullptr);
      ks = k > ks ? k : ks;
    }
    if (D % 256 == 0 && K % 128 == 0) {
      const int k = hr::launch_linear_mx(nullptr, nullptr, 0, nullptr, nullptr, T, D, K, HR_EPI_RESIDUAL, nullptr,
                                         nullptr, 0, nullptr, false, nullptr);
      ks = k > ks ? k : ks;
    }
  }
  return ks;
}

size_t ws_layout(const hr_dims* d, int32_t T, Ws* w, uint8_t* base) {
  const size_t D = d->hidden, F = d->ffn, A = size_t(d->n_q_heads) * d->head_dim;
  const size_t NQKV = size_t(d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
  const size_t t = size_t(T > 0 ? T : 0);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t* p = base ? base + off : nullptr;
    off += up256(bytes);
    return p;
  };
  Ws tmp;
  tmp.x = take(t * (D > A ? D : A) * 2);
  tmp.qkv = take(t * NQKV * 4);     // fp32: the q/k norm reads unrounded projections
  tmp.q = take(t * A * 2);
  tmp.attn = take(t * A * 2);
  tmp.act = take(t * F * 2);
  tmp.head = take(size_t(64) * D * 2);
  tmp.rope = reinterpret_cast<float*>(take(t * size_t(d->head_dim) * 4));
  // MXFP4 band: the codes reuse x (O / gate-up input) and act (down input)
  tmp.mx_ld = int((t + 255) / 256 * 256);
  tmp.mx_s1 = take(((D > A ? D : A) / 128) * size_t(tmp.mx_ld) * 4);
  tmp.mx_s2 = take((F / 128) * size_t(tmp.mx_ld) * 4);
  const int ks = residual_ks(d, T);
  tmp.part = ks > 1 ? reinterpret_cast<float*>(take(size_t(ks) * t * D * 4)) : nullptr;
  tmp.part_o = tmp.part_ml = nullptr;
  if (t > 0 && t <= size_t(kAttnSplitT)) {
    const size_t rows = part_rows(t);
    tmp.part_o = reinterpret_cast<float*>(take(rows * A * 4));
    tmp.part_ml = reinterpret_cast<float*>(take(rows * d->n_q_heads * 8));
  }
  tmp.k16 = tmp.v16 = nullptr;
  tmp.Tp = 0;
  if (hr::qkv_rope_fits(T, d->head_dim)) {
    tmp.Tp = (T + 31) / 32 * 32;
    const size_t bytes = size_t(tmp.Tp) * d->n_kv_heads * d->head_dim * 2;
    tmp.k16 = take(bytes);
    tmp.v16 = take(bytes);
  }
  if (w) *w = tmp;
  return off;
}

// Attention launch plan from the batch's host row lengths (start_pos + len).
// Key chunks: when the unsplit grid (query blocks x kv heads x sequences) is
// small against the CUs and the longest row is long, each query block takes 2
// or 4 key chunks of at least 8 tiles (64 keys each), the most that keep the
// grid within 512 workgroups; needs the partial buffers of the workspace (w).
// Measured (8 kv heads x 128, one query per stream after 2040 cached keys):
// 1 stream 44.6 -> 25.4 us, 8 streams 48.6 -> 29.1, 16 streams 49.2 -> 36.2
// (4 chunks), 32 streams 57.7 -> 51.8 (2 chunks); 8 chunks of 4 tiles were
// never faster by more than 5% and up to 1.6x slower (the combine step and
// the per-chunk start-up grow with the count); a prefill from position 0,
// 48 or more streams, or rows under 16 tiles run unsplit.  Two wave groups
// per block (interleaved key tiles) when the grid is still below one
// workgroup per CU and a block has at least 4 tiles.
// Every sequence one row (a decode step)?
bool one_row_batch(const hr_batch* b) {
  for (int s = 0; s < b->n_seq; ++s)
    if (b->h_cu_seqlens[s + 1] - b->h_cu_seqlens[s] != 1) return false;
  return true;
}

// Decode steps (one row per sequence) take decode_attention_kernel; with the
// workspace's partial buffers the keys are cut into chunks of ct 64-key tiles:
// the larger of 1/8 of the longest row and what keeps the grid (every chunk of
// every kv head of every stream) near kDecodeGrid workgroups; one chunk when
// that leaves fewer than 2.  Measured (8 kv heads x 128, µs; the rule's pick
// in brackets): 1 stream over 2041 keys 41.5 unsplit, [12.9] with 8 chunks of
// 4 tiles, 13.6 with 16 of 2; 16 streams 50.2 unsplit, [28.5] with 4 chunks of
// 8, 31.3 with 8 of 4; 32 streams [47.5] with 2 chunks, 52.0 unsplit; 64
// streams over 512 keys [25.2] unsplit, 33.6 with 2 chunks.
hr::AttnSplit decode_plan(const hr_dims* d, const hr_batch* b, const Ws* w) {
  hr::AttnSplit sp;
  sp.decode = true;
  if (!w || !w->part_o) return sp;
  long long units = 0;
  int max_tiles = 0;
  for (int s = 0; s < b->n_seq; ++s) {
    const int keys = d->causal ? b->h_start_pos[s] + 1 : b->h_used_keys[s];
    const int tiles = (keys + 63) / 64;
    units += (long long)tiles * d->n_kv_heads;
    if (tiles > max_tiles) max_tiles = tiles;
  }
  int ct = int((units + kDecodeGrid - 1) / kDecodeGrid);
  const int by_len = (max_tiles + kDecodeMaxSlots - 1) / kDecodeMaxSlots;
  if (ct < by_len) ct = by_len;
  if (ct < 1) ct = 1;
  const int want = (max_tiles + ct - 1) / ct;
  int cap = int(part_rows(size_t(b->total_tokens)) / size_t(b->total_tokens));
  if (cap > kDecodeMaxSlots) cap = kDecodeMaxSlots;
  if (want < 2 || cap < 2) return sp;
  sp.chunk_tiles = ct;
  sp.n_slots = want < cap ? want : cap;
  sp.part_o = w->part_o;
  sp.part_ml = w->part_ml;
  sp.T = b->total_tokens;
  return sp;
}

hr::AttnSplit attn_plan(const hr_dims* d, const hr_batch* b, const Ws* w) {
  if (one_row_batch(b)) return decode_plan(d, b, w);
  hr::AttnSplit sp;
  const int qpw = hr::attention_qpw(d->n_q_heads, d->n_kv_heads);
  long long wgs = 0;
  int max_keys = 0;
  for (int s = 0; s < b->n_seq; ++s) {
    const int len = b->h_cu_seqlens[s + 1] - b->h_cu_seqlens[s];
    wgs += (long long)((len + qpw - 1) / qpw) * d->n_kv_heads;
    const int keys = d->causal ? b->h_start_pos[s] + len : b->h_used_keys[s];
    if (keys > max_keys) max_keys = keys;
  }
  const int max_tiles = (max_keys + 63) / 64;
  int block_tiles = max_tiles;
  int slots = 1;
  for (int c = 2; c <= kAttnSlots; c *= 2)
    if (wgs * c <= kAttnSplitGrid && (max_tiles + c - 1) / c >= kAttnMinChunk) slots = c;
  if (w && w->part_o && slots > 1) {
    sp.chunk_tiles = kAttnChunk;
    sp.n_slots = slots;
    sp.part_o = w->part_o;
    sp.part_ml = w->part_ml;
    sp.T = b->total_tokens;
    wgs *= sp.n_slots;
    block_tiles = (max_tiles + sp.n_slots - 1) / sp.n_slots;
  }
  // a grid short of the 256 CUs splits each KV head's query heads over two
  // workgroups (P = 512, one sequence: 128 -> 256 workgroups)
  const int group = d->n_q_heads / d->n_kv_heads;
  if (wgs < 256 && group % 2 == 0) {
    sp.head_split = 2;
    wgs *= 2;
  }
  if (wgs < 512 && block_tiles >= 4) sp.groups = 2;
  return sp;
}

// The fused short-prompt path applies when every sequence starts at position
// 0 and has at most kSmallRows rows (its keys are its own rows): returns the
// longest sequence's rows then, else -1.
int small_prompt(const hr_batch* b) {
  int longest = 0;
  for (int s = 0; s < b->n_seq; ++s) {
    const int len = b->h_cu_seqlens[s + 1] - b->h_cu_seqlens[s];
    if (b->h_start_pos[s] != 0 || len > hr::kSmallRows) return -1;
    if (len > longest) longest = len;
  }
  return longest;
}

// Step A3 in the QKV GEMM's epilogue (hr::launch_qkv_rope) for batches that
// take the separate q/k-norm + RoPE step (not a decode step, not a short
// prompt) with 385-1024 rows: one launch and no fp32 QKV round trip instead of
// two (P = 512: the 8.4 us step).  Its angle table is built once per call.
bool qkv_rope_fused(const hr_dims* d, const hr_batch* b) {
  if (one_row_batch(b) && d->causal) return false;
  if (small_prompt(b) >= 0) return false;
  return hr::qkv_rope_fits(b->total_tokens, d->head_dim);
}

// Attention from the fp16 K / V copies that the fused QKV + step A3 launch
// writes (hr::launch_attention_f16): causal batches whose sequences all start
// at position 0 (their keys are their own rows) and at a row that is a
// multiple of 8.  Measured against the cache kernel (µs, 32 / 8 heads x 128):
// causal 400 rows 11.6 / 14.5, 512: 13.3 / 16.8, 2 x 256: 10.9 / 11.6, 640:
// 23.6 / 25.4, 1024: 29.2 / 31.4; non-causal 544 rows over 512 used keys
// 24.3 / 23.5 (no causal imbalance for the block pairs to even out), so
// non-causal batches keep the cache kernel and skip the copies.
bool attn_f16(const hr_dims* d, const hr_batch* b, const Ws& w, bool fused_qkv) {
  if (!fused_qkv || !w.k16 || !d->causal) return false;
  for (int s = 0; s < b->n_seq; ++s)
    if (b->h_start_pos[s] != 0 || b->h_cu_seqlens[s] % 8 != 0) return false;
  return true;
}

// The batch's RoPE angle table (workspace, built once per call) is read by
// the fused QKV epilogue and by the short-prompt RoPE + attention launch
// (whose workgroups otherwise compute their rows' angles in every layer).
bool rope_table_used(const hr_dims* d, const hr_batch* b) {
  if (one_row_batch(b) && d->causal) return false;   // decode steps: the decode launch
  return qkv_rope_fused(d, b) || small_prompt(b) >= 0;
}

// Input norm of a layer in its format: fp16 for the bf16 and MXFP4 bands
// (their QKV GEMM takes fp16 activations), e4m3 with the layer's QKV scale.
void in_norm_mode(const hr_layer* L, int* mode, float* inv) {
  const bool fp8 = L->wtype == HR_FP8_E4M3;
  *mode = fp8 ? hr::kNormE4M3 : hr::kNormF16;
  *inv = fp8 ? 1.0f / L->as_qkv : 1.f;
}

// one layer's kernels over buffers already validated.  `x_ready`: w.x already
// holds RMSNorm_in(h) of this layer.  `next`: the following layer (its input
// norm is fused with this layer's last residual add), or null: the residual
// is completed alone.
hr_status run_layer(const hr_dims* d, const hr_layer* L, const hr_layer* next, const hr_batch* b, float* h,
                    const hr_kv* kv, const Ws& w, bool x_ready, hipStream_t st) {
  const int T = b->total_tokens, D = d->hidden, F = d->ffn, Hq = d->n_q_heads, Hkv = d->n_kv_heads;
  const int dh = d->head_dim, A = Hq * dh, NQKV = (Hq + 2 * Hkv) * dh;
  const bool fp8 = L->wtype == HR_FP8_E4M3, mx = L->wtype == HR_MXFP4, pk = L->wtype == HR_F16_PACKED;
  const float eps = d->rms_eps;
  const hr::AttnSplit split = attn_plan(d, b, &w);
  if (!x_ready) {
    int mode;
    float inv;
    in_norm_mode(L, &mode, &inv);
    hr::launch_residual_norm(h, nullptr, 0, T, D, L->in_norm_w, eps, mode, w.x, inv, nullptr, nullptr, 0, st);
  }
  const bool fused_qkv = qkv_rope_fused(d, b);
  const bool f16_attn = attn_f16(d, b, w, fused_qkv);
  if (fused_qkv) {
    hr::QkvRope qr{w.q, kv->k, kv->v, b->cu_seqlens, b->start_pos, b->cache_slot, b->used_keys, b->n_seq,
                   d->causal, kv->capacity, Hq, Hkv, dh, L->q_norm_w, L->k_norm_w, eps, w.rope,
                   nullptr, nullptr, 0};
    if (f16_attn) {
      qr.k16 = w.k16;
      qr.v16 = w.v16;
      qr.Tp = w.Tp;
    }
    hr::launch_qkv_rope(w.x, L->w_qkv, L->ws_qkv, L->as_qkv, fp8, pk, T, D, qr, st);
  } else {
    hr::launch_linear(w.x, L->w_qkv, L->ws_qkv, L->as_qkv, fp8, pk, T, NQKV, D, HR_EPI_F32, w.qkv, 0.f, nullptr,
                      true, st);
  }
  if (split.decode && d->causal) {
    hr::launch_decode_rope_attention(w.qkv, L->q_norm_w, L->k_norm_w, d->rope_theta, eps, kv->k, kv->v,
                                     b->cu_seqlens, b->start_pos, b->cache_slot, b->n_seq, Hq, Hkv, dh,
                                     kv->capacity, w.attn, fp8, fp8 ? 1.0f / L->as_o : 1.f, split, st);
  } else if (const int small = small_prompt(b); small >= 0) {
    hr::launch_rope_attn_small(w.qkv, b->n_seq, small, Hq, Hkv, dh, d->rope_theta, eps, b->cu_seqlens,
                               b->cache_slot, b->used_keys, d->causal != 0, L->q_norm_w, L->k_norm_w, kv->k, kv->v,
                               kv->capacity, w.attn, fp8, fp8 ? 1.0f / L->as_o : 1.f, st, w.rope);
  } else {
    if (!fused_qkv)
      hr::launch_qknorm_rope_kv(w.qkv, T, Hq, Hkv, dh, d->rope_theta, eps, b->cu_seqlens, b->start_pos,
                                b->cache_slot, b->used_keys, b->n_seq, d->causal != 0, L->q_norm_w, L->k_norm_w,
                                w.q, kv->k, kv->v, kv->capacity, st);
    if (f16_attn)
      hr::launch_attention_f16(w.q, w.k16, w.v16, w.Tp, b->cu_seqlens, b->used_keys, b->n_seq, b->max_seqlen, Hq,
                               Hkv, dh, d->causal != 0, w.attn, fp8, fp8 ? 1.0f / L->as_o : 1.f, st);
    else
      hr::launch_attention(w.q, kv->k, kv->v, b->cu_seqlens, b->start_pos, b->cache_slot, b->used_keys, b->n_seq,
                           b->max_seqlen, Hq, Hkv, dh, kv->capacity, d->causal != 0, w.attn, fp8,
                           fp8 ? 1.0f / L->as_o : 1.f, st, &split);
  }
  // after the down projection: the residual completed, fused with the next
  // layer's input norm (or alone after the last layer)
  int next_mode = hr::kNormNone;
  float next_inv = 1.f;
  if (next) in_norm_mode(next, &next_mode, &next_inv);
  const void* next_w = next ? next->in_norm_w : nullptr;
  if (mx) {
    // O, gate/up and down on MXFP4: per-row block quantisation of each input
    // (1/s applied first), the gate/up epilogue writing the down input
    const uint8_t* wo = static_cast<const uint8_t*>(L->w_o);
    hr::launch_quant_mx(w.attn, 2, T, A, L->awq_inv_o, nullptr, w.x, w.mx_s1, w.mx_ld, st);
    int ks = hr::launch_linear_mx(w.x, w.mx_s1, w.mx_ld, wo, L->mx_o_s, T, D, A, HR_EPI_RESIDUAL, h, nullptr, 0,
                                  w.part, true, st);
    hr::launch_residual_norm(h, w.part, ks > 1 ? ks : 0, T, D, L->post_norm_w, eps, hr::kNormMX, w.x, 1.f,
                             L->awq_inv_gu, w.mx_s1, w.mx_ld, st);
    hr::launch_linear_mx(w.x, w.mx_s1, w.mx_ld, static_cast<const uint8_t*>(L->w_gu), L->mx_gu_s, T, 2 * F, D,
                         HR_EPI_SWIGLU, w.act, w.mx_s2, w.mx_ld, nullptr, true, st);
    ks = hr::launch_linear_mx(w.act, w.mx_s2, w.mx_ld, static_cast<const uint8_t*>(L->w_down), L->mx_down_s, T, D,
                              F, HR_EPI_RESIDUAL, h, nullptr, 0, w.part, true, st);
    hr::launch_residual_norm(h, w.part, ks > 1 ? ks : 0, T, D, next_w, eps, next_mode, w.x, next_inv, nullptr,
                             nullptr, 0, st);
    return check_launch("prefill layer (MXFP4)");
  }
  int ks = hr::launch_linear(w.attn, L->w_o, L->ws_o, L->as_o, fp8, pk, T, D, A, HR_EPI_RESIDUAL, h, 0.f, w.part,
                             true, st);
  hr::launch_residual_norm(h, w.part, ks > 1 ? ks : 0, T, D, L->post_norm_w, eps,
                           fp8 ? hr::kNormE4M3 : hr::kNormF16, w.x, fp8 ? 1.0f / L->as_gu : 1.f, nullptr, nullptr, 0,
                           st);
  hr::launch_linear(w.x, L->w_gu, L->ws_gu, L->as_gu, fp8, pk, T, 2 * F, D, HR_EPI_SWIGLU, w.act,
                    fp8 ? L->as_down : 0.f, nullptr, true, st);
  ks = hr::launch_linear(w.act, L->w_down, L->ws_down, L->as_down, fp8, pk, T, D, F, HR_EPI_RESIDUAL, h, 0.f,
                         w.part, true, st);
  hr::launch_residual_norm(h, w.part, ks > 1 ? ks : 0, T, D, next_w, eps, next_mode, w.x, next_inv, nullptr, nullptr,
                           0, st);
  return check_launch("prefill layer");
}

hr_status run_head(const float* h, const hr_batch* b, int D, const void* final_w, float eps,
                   const void* head_w, int K, int V, float* logits, void* zbuf, hipStream_t st) {
  const int N = K * V;
  for (int s0 = 0; s0 < b->n_seq; s0 += 32) {
    const int n = (b->n_seq - s0) < 32 ? (b->n_seq - s0) : 32;
    hr::launch_final_split(h, b->cu_seqlens, s0, n, D, final_w, eps, n, zbuf, st);
    hr::launch_head_gemm(zbuf, n, head_w, N, D, logits + size_t(s0) * N, st);
  }
  return check_launch("head");
}

}  // namespace

extern "C" {

const char* hr_last_error(void) { return g_err.c_str(); }

size_t hr_workspace_bytes(const hr_dims* dims, hr_wtype wtype, int32_t total_tokens) {
  (void)wtype;
  if (!dims || total_tokens < 0) return 0;
  return ws_layout(dims, total_tokens, nullptr, nullptr);
}

hr_status hr_prefill_layer(const hr_dims* dims, const hr_layer* layer, const hr_batch* batch, float* h,
                           const hr_kv* kv, void* ws, size_t ws_bytes, hipStream_t stream) {
  HR_TRY(check_dims(dims));
  HR_TRY(check_layer(dims, layer, 0));
  HR_TRY(check_kv(dims, kv, "kv"));
  HR_TRY(check_batch(dims, batch, kv));
  if (batch->total_tokens == 0) return HR_OK;
  HR_TRY(need(h, "h"));
  HR_TRY(need(ws, "ws"));
  const size_t need_ws = ws_layout(dims, batch->total_tokens, nullptr, nullptr);
  if (ws_bytes < need_ws) return fail(HR_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need_ws);
  Ws w;
  ws_layout(dims, batch->total_tokens, &w, static_cast<uint8_t*>(ws));
  if (rope_table_used(dims, batch))
    hr::launch_rope_table(batch->cu_seqlens, batch->start_pos, batch->n_seq, batch->total_tokens, dims->head_dim,
                          dims->rope_theta, w.rope, stream);
  return run_layer(dims, layer, nullptr, batch, h, kv, w, false, stream);
}

}  // extern "C"

namespace {

// every check of hr_prefill_stack, before anything is launched
hr_status check_stack(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch, const int32_t* ids,
                      const void* embed, int32_t vocab, const void* x_embeds, const hr_kv* kv,
                      const void* final_norm_w, const void* head_w, int32_t n_codebooks, int32_t cb_vocab,
                      const float* logits_out) {
  HR_TRY(check_dims(dims));
  if (dims->n_layers <= 0) return fail(HR_EINVAL, "n_layers must be > 0");
  if (!layers || !kv) return fail(HR_EINVAL, "layers and kv arrays are required");
  for (int l = 0; l < dims->n_layers; ++l) {
    HR_TRY(check_layer(dims, &layers[l], l));
    if (layers[l].wtype != layers[0].wtype) return fail(HR_EINVAL, "all layers must share one wtype");
    HR_TRY(check_kv(dims, &kv[l], "kv[l]"));
    HR_TRY(check_batch(dims, batch, &kv[l]));
  }
  if (ids) {
    HR_TRY(need(embed, "embed"));
    if (vocab <= 0) return fail(HR_EINVAL, "vocab must be > 0");
  } else {
    HR_TRY(need(x_embeds, "x_embeds (ids is NULL)"));
  }
  HR_TRY(need(final_norm_w, "final_norm_w"));
  if ((head_w != nullptr) != (logits_out != nullptr))
    return fail(HR_EINVAL, "head_w and logits_out must both be given or both NULL");
  if (head_w) {
    HR_TRY(need(head_w, "head_w"));
    HR_TRY(need(logits_out, "logits_out"));
    if (n_codebooks <= 0 || cb_vocab <= 0) return fail(HR_EINVAL, "n_codebooks and cb_vocab must be > 0");
    for (int s = 0; s < batch->n_seq; ++s)
      if (batch->h_cu_seqlens[s + 1] <= batch->h_cu_seqlens[s])
        return fail(HR_EINVAL, "sequence %d is empty: no last row for the head", s);
  }
  return HR_OK;
}

// the stack's kernels over validated arguments and a laid-out workspace
hr_status enqueue_stack(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch, const int32_t* ids,
                        const void* embed, const void* x_embeds, const hr_kv* kv, const void* final_norm_w,
                        const void* head_w, int32_t n_codebooks, int32_t cb_vocab, float* h_out,
                        float* logits_out, const Ws& w, hipStream_t stream) {
  const int T = batch->total_tokens, D = dims->hidden;
  const hr_layer& L0 = layers[0];
  const bool fp8 = L0.wtype == HR_FP8_E4M3;
  hr::launch_embed_rmsnorm(ids, embed, x_embeds, T, D, L0.in_norm_w, dims->rms_eps, h_out, w.x, fp8,
                           fp8 ? 1.0f / L0.as_qkv : 1.f, stream);
  if (rope_table_used(dims, batch))   // the angles are the same for every layer
    hr::launch_rope_table(batch->cu_seqlens, batch->start_pos, batch->n_seq, T, dims->head_dim, dims->rope_theta,
                          w.rope, stream);
  // every layer's input norm after the first is fused into the previous
  // layer's last residual add
  for (int l = 0; l < dims->n_layers; ++l)
    HR_TRY(run_layer(dims, &layers[l], l + 1 < dims->n_layers ? &layers[l + 1] : nullptr, batch, h_out, &kv[l], w,
                     true, stream));
  if (head_w)
    HR_TRY(run_head(h_out, batch, D, final_norm_w, dims->rms_eps, head_w, n_codebooks, cb_vocab, logits_out,
                    w.head, stream));
  return check_launch("prefill stack");
}

// every check of hr_codebook_step
hr_status check_codebook(int32_t B, int32_t K, int32_t V, int32_t bos_id, int32_t eoc_id, const void* logits,
                         const int32_t* frame, const uint8_t* eoc_seen, const uint8_t* done, const int32_t* codes,
                         const int32_t* aligned, int32_t max_frames, const void* cb_embed, int32_t D,
                         const void* emb_out) {
  if (B < 0 || K <= 0 || V < 2 || D <= 0) return fail(HR_EINVAL, "bad sizes B=%d K=%d V=%d D=%d", B, K, V, D);
  if (K > 1024) return fail(HR_EUNSUPPORTED, "K = %d > 1024 codebooks", K);
  if (D % 8) return fail(HR_EINVAL, "D = %d is not a multiple of 8", D);
  if (bos_id < 0 || bos_id >= V || eoc_id < 0 || eoc_id >= V || bos_id == eoc_id)
    return fail(HR_EINVAL, "bos_id %d / eoc_id %d must be distinct ids in [0, %d)", bos_id, eoc_id, V);
  if (!logits || !frame || !eoc_seen || !done || !codes) return fail(HR_EINVAL, "NULL state pointer");
  HR_TRY(need(logits, "logits"));
  if (aligned && max_frames <= 0) return fail(HR_EINVAL, "max_frames must be > 0 when aligned is given");
  HR_TRY(need(cb_embed, "cb_embed"));
  HR_TRY(need(emb_out, "emb_out"));
  return HR_OK;
}

// decode workspace: the prefill workspace of B rows, then h fp32 [B, D]
size_t decode_ws_layout(const hr_dims* d, int32_t B, Ws* w, float** h, uint8_t* base) {
  const size_t off = ws_layout(d, B, w, base);
  if (h) *h = base ? reinterpret_cast<float*>(base + off) : nullptr;
  return off + up256(size_t(B) * d->hidden * 4);
}

}  // namespace

extern "C" {

hr_status hr_prefill_stack(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch,
                           const int32_t* ids, const void* embed, int32_t vocab, const void* x_embeds,
                           const hr_kv* kv, const void* final_norm_w, const void* head_w,
                           int32_t n_codebooks, int32_t cb_vocab, float* h_out, float* logits_out,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  HR_TRY(check_stack(dims, layers, batch, ids, embed, vocab, x_embeds, kv, final_norm_w, head_w, n_codebooks,
                     cb_vocab, logits_out));
  if (batch->total_tokens == 0) return HR_OK;
  HR_TRY(need(h_out, "h_out"));
  HR_TRY(need(ws, "ws"));
  const size_t need_ws = ws_layout(dims, batch->total_tokens, nullptr, nullptr);
  if (ws_bytes < need_ws) return fail(HR_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need_ws);
  Ws w;
  ws_layout(dims, batch->total_tokens, &w, static_cast<uint8_t*>(ws));
  return enqueue_stack(dims, layers, batch, ids, embed, x_embeds, kv, final_norm_w, head_w, n_codebooks, cb_vocab,
                       h_out, logits_out, w, stream);
}

size_t hr_decode_workspace_bytes(const hr_dims* dims, hr_wtype wtype, int32_t B) {
  (void)wtype;
  if (!dims || B < 0) return 0;
  return decode_ws_layout(dims, B, nullptr, nullptr, nullptr);
}

}  // extern "C"

namespace {

// every check of a decode step except the workspace's
hr_status check_decode(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch, const void* x_embeds,
                       const hr_kv* kv, const void* final_norm_w, const void* head_w, int32_t n_codebooks,
                       int32_t cb_vocab, int32_t bos_id, int32_t eoc_id, float* logits_out, int32_t* frame,
                       uint8_t* eoc_seen, uint8_t* done, int32_t* codes, int32_t* aligned, int32_t max_frames,
                       const void* cb_embed, void* emb_out) {
  if (!dims) return fail(HR_EINVAL, "dims is NULL");
  if (!dims->causal) return fail(HR_EUNSUPPORTED, "a decode step attends causally (dims->causal = 0)");
  if (!batch) return fail(HR_EINVAL, "batch is NULL");
  if (!head_w || !logits_out) return fail(HR_EINVAL, "a decode step needs head_w and logits_out");
  HR_TRY(check_stack(dims, layers, batch, nullptr, nullptr, 0, x_embeds, kv, final_norm_w, head_w, n_codebooks,
                     cb_vocab, logits_out));
  const int B = batch->n_seq;
  if (batch->total_tokens != B)
    return fail(HR_EINVAL, "a decode step takes one row per stream (total_tokens %d, n_seq %d)",
                batch->total_tokens, B);
  for (int s = 0; s < B; ++s)
    if (batch->h_cu_seqlens[s + 1] - batch->h_cu_seqlens[s] != 1)
      return fail(HR_EINVAL, "stream %d has %d rows; a decode step takes one", s,
                  batch->h_cu_seqlens[s + 1] - batch->h_cu_seqlens[s]);
  HR_TRY(check_codebook(B, n_codebooks, cb_vocab, bos_id, eoc_id, logits_out, frame, eoc_seen, done, codes,
                        aligned, max_frames, cb_embed, dims->hidden, emb_out));
  return HR_OK;
}

// the decode step's kernels over validated arguments and a large enough workspace
hr_status enqueue_decode(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch, const void* x_embeds,
                         const hr_kv* kv, const void* final_norm_w, const void* head_w, int32_t n_codebooks,
                         int32_t cb_vocab, int32_t bos_id, int32_t eoc_id, float* logits_out, int32_t* frame,
                         uint8_t* eoc_seen, uint8_t* done, int32_t* codes, int32_t* aligned, int32_t max_frames,
                         const void* cb_embed, void* emb_out, void* ws, hipStream_t stream) {
  const int B = batch->n_seq;
  Ws w;
  float* h = nullptr;
  decode_ws_layout(dims, B, &w, &h, static_cast<uint8_t*>(ws));
  HR_TRY(enqueue_stack(dims, layers, batch, nullptr, nullptr, x_embeds, kv, final_norm_w, head_w, n_codebooks,
                       cb_vocab, h, logits_out, w, stream));
  hr::launch_codebook_step(B, n_codebooks, cb_vocab, bos_id, eoc_id, true, logits_out, frame, eoc_seen, done,
                           codes, aligned, max_frames, cb_embed, dims->hidden, emb_out, stream);
  return check_launch("decode step");
}

// Scratch of hr_decode_step_noalloc: a file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  In host code
// `scratch` names a host-side stand-in, never the device memory: its address
// on a device comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(32) << 20;   // 4B-class decode steps of up to 128 streams (27 MiB)
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hr_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HR_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HR_EUNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(HR_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HR_OK;
}

}  // namespace

extern "C" {

hr_status hr_decode_step(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch, const void* x_embeds,
                         const hr_kv* kv, const void* final_norm_w, const void* head_w, int32_t n_codebooks,
                         int32_t cb_vocab, int32_t bos_id, int32_t eoc_id, float* logits_out, int32_t* frame,
                         uint8_t* eoc_seen, uint8_t* done, int32_t* codes, int32_t* aligned, int32_t max_frames,
                         const void* cb_embed, void* emb_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  HR_TRY(check_decode(dims, layers, batch, x_embeds, kv, final_norm_w, head_w, n_codebooks, cb_vocab, bos_id, eoc_id,
                      logits_out, frame, eoc_seen, done, codes, aligned, max_frames, cb_embed, emb_out));
  HR_TRY(need(ws, "ws"));
  const size_t need_ws = decode_ws_layout(dims, batch->n_seq, nullptr, nullptr, nullptr);
  if (ws_bytes < need_ws) return fail(HR_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need_ws);
  return enqueue_decode(dims, layers, batch, x_embeds, kv, final_norm_w, head_w, n_codebooks, cb_vocab, bos_id,
                        eoc_id, logits_out, frame, eoc_seen, done, codes, aligned, max_frames, cb_embed, emb_out, ws,
                        stream);
}

size_t hr_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

hr_status hr_decode_step_noalloc(const hr_dims* dims, const hr_layer* layers, const hr_batch* batch,
                                 const void* x_embeds, const hr_kv* kv, const void* final_norm_w, const void* head_w,
                                 int32_t n_codebooks, int32_t cb_vocab, int32_t bos_id, int32_t eoc_id,
                                 float* logits_out, int32_t* frame, uint8_t* eoc_seen, uint8_t* done, int32_t* codes,
                                 int32_t* aligned, int32_t max_frames, const void* cb_embed, void* emb_out,
                                 hipStream_t stream) {
  HR_TRY(check_decode(dims, layers, batch, x_embeds, kv, final_norm_w, head_w, n_codebooks, cb_vocab, bos_id, eoc_id,
                      logits_out, frame, eoc_seen, done, codes, aligned, max_frames, cb_embed, emb_out));
  const size_t need_ws = decode_ws_layout(dims, batch->n_seq, nullptr, nullptr, nullptr);
  if (need_ws > kScratchBytes)
    return fail(HR_EWORKSPACE, "a decode step of %d streams needs %zu bytes of scratch; the allocation-free entry "
                "holds %zu (hr_decode_step with a caller workspace has no such limit)",
                batch->n_seq, need_ws, kScratchBytes);
  void* ws = nullptr;
  HR_TRY(scratch_of_current_device(&ws));
  // every scratch region is written before it is read within the call
  // (split-K partials, attention partials, activations), so nothing is cleared
  return enqueue_decode(dims, layers, batch, x_embeds, kv, final_norm_w, head_w, n_codebooks, cb_vocab, bos_id,
                        eoc_id, logits_out, frame, eoc_seen, done, codes, aligned, max_frames, cb_embed, emb_out, ws,
                        stream);
}

hr_status hr_codebook_step(int32_t B, int32_t K, int32_t V, int32_t bos_id, int32_t eoc_id,
                           int32_t logits_is_fp32, const void* logits, int32_t* frame, uint8_t* eoc_seen,
                           uint8_t* done, int32_t* codes, int32_t* aligned, int32_t max_frames,
                           const void* cb_embed, int32_t D, void* emb_out, hipStream_t stream) {
  HR_TRY(check_codebook(B, K, V, bos_id, eoc_id, logits, frame, eoc_seen, done, codes, aligned, max_frames,
                        cb_embed, D, emb_out));
  if (B == 0) return HR_OK;
  hr::launch_codebook_step(B, K, V, bos_id, eoc_id, logits_is_fp32 != 0, logits, frame, eoc_seen, done, codes,
                           aligned, max_frames, cb_embed, D, emb_out, stream);
  return check_launch("codebook step");
}

hr_status hr_codebook_step_policy(int32_t B, int32_t K, int32_t V, int32_t bos_id, int32_t eoc_id,
                                  int32_t logits_is_fp32, const void* logits, int32_t* frame, uint8_t* eoc_seen,
                                  uint8_t* done, int32_t* codes, int32_t* aligned, int32_t max_frames,
                                  const void* cb_embed, int32_t D, void* emb_out, const hr_step_policy* policy,
                                  hipStream_t stream) {
  HR_TRY(check_codebook(B, K, V, bos_id, eoc_id, logits, frame, eoc_seen, done, codes, aligned, max_frames,
                        cb_embed, D, emb_out));
  if (V > 2048) return fail(HR_EUNSUPPORTED, "V = %d > 2048 ids per codebook for the policy step", V);
  hr::StepPolicy p;
  if (policy) {
    p.temperature = policy->temperature;
    p.top_k = policy->top_k;
    p.top_p = policy->top_p;
    p.seed = policy->seed;
    p.eoc_cascade = policy->eoc_cascade != 0;
    p.repeat_limit = policy->repeat_limit;
    p.end_frame = policy->end_frame;
    p.last_codes = policy->last_codes;
    p.repeat_run = policy->repeat_run;
    if (p.temperature && !p.seed) return fail(HR_EINVAL, "temperature given without seed");
    if (p.seed && (reinterpret_cast<uintptr_t>(p.seed) & 7))
      return fail(HR_EALIGN, "seed is not 8-byte aligned");
    if (p.repeat_limit < 0 || p.repeat_limit == 1)
      return fail(HR_EINVAL, "repeat_limit %d: 0 (off) or >= 2", p.repeat_limit);
    if ((p.eoc_cascade || p.repeat_limit) && !p.end_frame)
      return fail(HR_EINVAL, "end_frame is required by the cascade and the stop guard");
    if (p.repeat_limit && (!p.last_codes || !p.repeat_run))
      return fail(HR_EINVAL, "last_codes and repeat_run are required by the stop guard");
  }
  if (B == 0) return HR_OK;
  if (!p.temperature && !p.eoc_cascade && !p.repeat_limit)   // greedy, no policy: the plain step's kernel
    hr::launch_codebook_step(B, K, V, bos_id, eoc_id, logits_is_fp32 != 0, logits, frame, eoc_seen, done, codes,
                             aligned, max_frames, cb_embed, D, emb_out, stream);
  else
    hr::launch_codebook_policy(B, K, V, bos_id, eoc_id, logits_is_fp32 != 0, logits, frame, eoc_seen, done, codes,
                               aligned, max_frames, cb_embed, D, emb_out, p, stream);
  return check_launch("codebook policy step");
}

// ------------------------------------------------------------------ step-level entries (hr_ops.h)
hr_status hr_embed_rmsnorm(const int32_t* ids, const void* embed, int32_t vocab, const void* x_embeds,
                           int32_t T, int32_t D, const void* norm_w, float eps, float* h_out, void* x_out,
                           hr_wtype x_type, float x_scale, hipStream_t stream) {
  if (T < 0 || D <= 0 || D % 8 || D > 8192) return fail(HR_EINVAL, "bad T=%d / D=%d", T, D);
  if (ids) {
    HR_TRY(need(embed, "embed"));
    if (vocab <= 0) return fail(HR_EINVAL, "vocab must be > 0");
  } else {
    HR_TRY(need(x_embeds, "x_embeds"));
  }
  HR_TRY(need(norm_w, "norm_w"));
  HR_TRY(need(h_out, "h_out"));
  HR_TRY(need(x_out, "x_out"));
  if (x_type != HR_F16 && x_type != HR_FP8_E4M3) return fail(HR_EINVAL, "x_type: HR_F16 or HR_FP8_E4M3");
  if (x_type == HR_FP8_E4M3 && !(x_scale > 0.f)) return fail(HR_EINVAL, "x_scale must be > 0");
  if (T == 0) return HR_OK;
  hr::launch_embed_rmsnorm(ids, embed, x_embeds, T, D, norm_w, eps, h_out, x_out, x_type == HR_FP8_E4M3,
                           x_type == HR_FP8_E4M3 ? 1.0f / x_scale : 1.f, stream);
  return check_launch("embed_rmsnorm");
}

hr_status hr_rmsnorm(const float* h, int32_t T, int32_t D, const void* norm_w, float eps, void* x_out,
                     hr_wtype x_type, float x_scale, hipStream_t stream) {
  if (T < 0 || D <= 0 || D % 8 || D > 8192) return fail(HR_EINVAL, "bad T=%d / D=%d", T, D);
  HR_TRY(need(h, "h"));
  HR_TRY(need(norm_w, "norm_w"));
  HR_TRY(need(x_out, "x_out"));
  if (x_type != HR_F16 && x_type != HR_FP8_E4M3) return fail(HR_EINVAL, "x_type: HR_F16 or HR_FP8_E4M3");
  if (x_type == HR_FP8_E4M3 && !(x_scale > 0.f)) return fail(HR_EINVAL, "x_scale must be > 0");
  if (T == 0) return HR_OK;
  hr::launch_rmsnorm(h, T, D, norm_w, eps, x_out, x_type == HR_FP8_E4M3,
                     x_type == HR_FP8_E4M3 ? 1.0f / x_scale : 1.f, stream);
  return check_launch("rmsnorm");
}

size_t hr_linear_workspace_bytes(hr_wtype wtype, int32_t M, int32_t N, int32_t K, hr_epilogue epi) {
  if (epi != HR_EPI_RESIDUAL || M <= 0 || N <= 0 || K <= 0) return 0;
  int ks = 1;
  if (wtype == HR_MXFP4) {
    if (K % 128) return 0;
    ks = hr::launch_linear_mx(nullptr, nullptr, 0, nullptr, nullptr, M, N, K, HR_EPI_RESIDUAL, nullptr, nullptr, 0,
                              nullptr, false, nullptr);
  } else {
    const bool fp8 = wtype == HR_FP8_E4M3, pk = wtype == HR_F16_PACKED;
    if (K % (fp8 ? 128 : 64)) return 0;
    // the plan of the format that will run (its split factor sizes the partials)
    ks = hr::launch_linear(nullptr, nullptr, nullptr, 1.f, fp8, pk, M, N, K, HR_EPI_RESIDUAL, nullptr, 0.f,
                           nullptr, false, nullptr);
  }
  return ks > 1 ? up256(size_t(ks) * size_t(M) * size_t(N) * 4) : 0;
}

hr_status hr_linear(const void* x, const void* w, const float* w_scale, float x_scale, hr_wtype wtype,
                    int32_t M, int32_t N, int32_t K, hr_epilogue epi, void* out, float out_scale, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  if (M < 0 || N <= 0 || K <= 0) return fail(HR_EINVAL, "bad M=%d N=%d K=%d", M, N, K);
  if (epi != HR_EPI_F32 && epi != HR_EPI_RESIDUAL && epi != HR_EPI_SWIGLU) return fail(HR_EINVAL, "bad epilogue");
  if (wtype != HR_BF16 && wtype != HR_FP8_E4M3 && wtype != HR_F16_PACKED) return fail(HR_EINVAL, "bad wtype");
  const bool fp8 = wtype == HR_FP8_E4M3, pk = wtype == HR_F16_PACKED;
  if (K % (fp8 ? 128 : 64)) return fail(HR_EUNSUPPORTED, "K = %d must be a multiple of %d", K, fp8 ? 128 : 64);
  if (uint64_t(M > N ? M : N) * K * (fp8 ? 1 : 2) >= (uint64_t(1) << 32))
    return fail(HR_EUNSUPPORTED, "an operand of %d x %d or %d x %d exceeds 4 GB", M, K, N, K);
  if (N % 16 || (epi == HR_EPI_SWIGLU && N % 32))
    return fail(HR_EUNSUPPORTED, "N = %d must be a multiple of 16 (32 for SwiGLU)", N);
  if (pk && epi == HR_EPI_SWIGLU && N % 64)
    return fail(HR_EUNSUPPORTED, "packed gate/up: N = %d must be a multiple of 64", N);
  HR_TRY(need(x, "x"));
  HR_TRY(need(w, "w"));
  HR_TRY(need(out, "out"));
  if (fp8) {
    if (!w_scale) return fail(HR_EINVAL, "FP8 needs w_scale");
    if (!(x_scale > 0.f)) return fail(HR_EINVAL, "FP8 needs x_scale > 0");
    if (epi == HR_EPI_SWIGLU && !(out_scale > 0.f)) return fail(HR_EINVAL, "FP8 SwiGLU needs out_scale > 0");
  }
  const size_t need_ws = hr_linear_workspace_bytes(wtype, M, N, K, epi);
  if (need_ws) {
    if (!ws || ws_bytes < need_ws)
      return fail(HR_EWORKSPACE, "linear workspace needs %zu bytes, got %zu", need_ws, ws ? ws_bytes : size_t(0));
    HR_TRY(need(ws, "ws"));
  }
  if (M == 0) return HR_OK;
  const int ks = hr::launch_linear(x, w, w_scale, x_scale, fp8, pk, M, N, K, epi, out, out_scale,
                                   static_cast<float*>(ws), true, stream);
  if (epi == HR_EPI_RESIDUAL && ks > 1)
    hr::launch_residual_sum(static_cast<float*>(out), static_cast<const float*>(ws), ks, size_t(M) * size_t(N),
                            stream);
  return check_launch("linear");
}

hr_status hr_pack_weight(const void* w, int32_t N, int32_t K, int32_t gate_up, void* out, hipStream_t stream) {
  if (N <= 0 || K <= 0 || K % 32) return fail(HR_EINVAL, "bad N=%d / K=%d (K a multiple of 32)", N, K);
  if (gate_up != 0 && gate_up != 1) return fail(HR_EINVAL, "gate_up must be 0 or 1");
  if (gate_up && N % 64) return fail(HR_EUNSUPPORTED, "gate/up: N = 2F = %d must be a multiple of 64", N);
  if (uint64_t(N) * uint64_t(K) * 2 >= (uint64_t(1) << 31))
    return fail(HR_EUNSUPPORTED, "a %d x %d weight exceeds 2 GB", N, K);
  HR_TRY(need(w, "w"));
  HR_TRY(need(out, "out"));
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), o = reinterpret_cast<uintptr_t>(out);
  const uintptr_t bytes = uintptr_t(N) * uintptr_t(K) * 2;
  if (a < o + bytes && o < a + bytes) return fail(HR_EINVAL, "out overlaps w");
  const int rc = hr::launch_pack_weight(w, N, K, gate_up != 0, out, stream);
  if (rc < 0) return fail(HR_EHIP, "pack weight: %s", hipGetErrorString(hipGetLastError()));
  if (rc > 0) return fail(HR_EINVAL, "a weight is outside the fp16 range (|w| >= 65520, inf or NaN)");
  return HR_OK;
}

hr_status hr_residual_rmsnorm(float* h, const float* partials, int32_t n_partials, int32_t T, int32_t D,
                              const void* norm_w, float eps, void* x_out, hr_wtype x_type, float x_scale,
                              hipStream_t stream) {
  if (T < 0 || D <= 0 || D % 8 || D > 8192) return fail(HR_EINVAL, "bad T=%d / D=%d", T, D);
  if (n_partials < 0) return fail(HR_EINVAL, "n_partials %d < 0", n_partials);
  HR_TRY(need(h, "h"));
  if (n_partials > 0) HR_TRY(need(partials, "partials"));
  if (x_out) {
    HR_TRY(need(x_out, "x_out"));
    HR_TRY(need(norm_w, "norm_w"));
    if (x_type != HR_F16 && x_type != HR_FP8_E4M3) return fail(HR_EINVAL, "x_type: HR_F16 or HR_FP8_E4M3");
    if (x_type == HR_FP8_E4M3 && !(x_scale > 0.f)) return fail(HR_EINVAL, "x_scale must be > 0");
  }
  if (T == 0) return HR_OK;
  const int mode = !x_out ? hr::kNormNone : (x_type == HR_FP8_E4M3 ? hr::kNormE4M3 : hr::kNormF16);
  hr::launch_residual_norm(h, partials, n_partials, T, D, norm_w, eps, mode, x_out,
                           x_type == HR_FP8_E4M3 ? 1.0f / x_scale : 1.f, nullptr, nullptr, 0, stream);
  return check_launch("residual_rmsnorm");
}

hr_status hr_quantize_mxfp4(const void* x, int32_t x_format, int32_t M, int32_t K, const float* col_scale,
                            const float* row_scale, uint8_t* codes, uint8_t* scales, int32_t ld_scales,
                            hipStream_t stream) {
  if (M < 0 || K <= 0 || K % 128) return fail(HR_EINVAL, "bad M=%d / K=%d (a multiple of 128)", M, K);
  if (ld_scales < M || ld_scales % 4) return fail(HR_EINVAL, "ld_scales %d: >= M and a multiple of 4", ld_scales);
  if (x_format < 0 || x_format > 2) return fail(HR_EINVAL, "x_format %d: 0 bf16, 1 fp32, 2 fp16", x_format);
  HR_TRY(need(x, "x"));
  HR_TRY(need(codes, "codes"));
  HR_TRY(need(scales, "scales"));
  if (col_scale && !aligned16(col_scale)) return fail(HR_EALIGN, "col_scale is not 16-byte aligned");
  if (M == 0) return HR_OK;
  hr::launch_quant_mx(x, x_format, M, K, col_scale, row_scale, codes, scales, ld_scales, stream);
  return check_launch("quantize mxfp4");
}

hr_status hr_rmsnorm_mxfp4(const float* h, int32_t T, int32_t D, const void* norm_w, float eps,
                           const float* col_scale, uint8_t* codes, uint8_t* scales, int32_t ld_scales,
                           hipStream_t stream) {
  if (T < 0 || D <= 0 || D % 128 || D > 8192) return fail(HR_EINVAL, "bad T=%d / D=%d", T, D);
  if (ld_scales < T || ld_scales % 4) return fail(HR_EINVAL, "ld_scales %d: >= T and a multiple of 4", ld_scales);
  HR_TRY(need(h, "h"));
  HR_TRY(need(norm_w, "norm_w"));
  HR_TRY(need(codes, "codes"));
  HR_TRY(need(scales, "scales"));
  if (col_scale && !aligned16(col_scale)) return fail(HR_EALIGN, "col_scale is not 16-byte aligned");
  if (T == 0) return HR_OK;
  hr::launch_rmsnorm_mx(h, T, D, norm_w, col_scale, eps, codes, scales, ld_scales, stream);
  return check_launch("rmsnorm mxfp4");
}

hr_status hr_linear_mxfp4(const uint8_t* x, const uint8_t* x_scales, int32_t ld_x_scales, const uint8_t* w,
                          const uint8_t* w_scales, int32_t M, int32_t N, int32_t K, hr_epilogue epi, void* out,
                          uint8_t* out_scales, int32_t ld_out_scales, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  if (M < 0 || N <= 0 || K <= 0 || K % 128) return fail(HR_EINVAL, "bad M=%d N=%d K=%d (K a multiple of 128)", M, N, K);
  if (epi != HR_EPI_RESIDUAL && epi != HR_EPI_SWIGLU) return fail(HR_EINVAL, "MXFP4: residual or SwiGLU epilogue");
  if (epi == HR_EPI_RESIDUAL && N % 256) return fail(HR_EUNSUPPORTED, "N = %d must be a multiple of 256", N);
  if (epi == HR_EPI_SWIGLU && N % 256) return fail(HR_EUNSUPPORTED, "N = 2F = %d: F a multiple of 128", N);
  const int32_t Mr = (M + 255) / 256 * 256;
  if (ld_x_scales < Mr || ld_x_scales % 4) return fail(HR_EINVAL, "ld_x_scales %d < %d", ld_x_scales, Mr);
  if (uint64_t(M > N ? M : N) * (K / 2) >= (uint64_t(1) << 31))
    return fail(HR_EUNSUPPORTED, "an operand of %d x %d or %d x %d exceeds 2 GB", M, K, N, K);
  HR_TRY(need(x, "x"));
  HR_TRY(need(x_scales, "x_scales"));
  HR_TRY(need(w, "w"));
  HR_TRY(need(w_scales, "w_scales"));
  HR_TRY(need(out, "out"));
  if (epi == HR_EPI_SWIGLU) {
    HR_TRY(need(out_scales, "out_scales"));
    if (ld_out_scales < Mr || ld_out_scales % 4)
      return fail(HR_EINVAL, "ld_out_scales %d < %d", ld_out_scales, Mr);
  }
  const size_t need_ws = hr_linear_workspace_bytes(HR_MXFP4, M, N, K, epi);
  if (need_ws) {
    if (!ws || ws_bytes < need_ws)
      return fail(HR_EWORKSPACE, "linear workspace needs %zu bytes, got %zu", need_ws, ws ? ws_bytes : size_t(0));
    HR_TRY(need(ws, "ws"));
  }
  if (M == 0) return HR_OK;
  const int ks = hr::launch_linear_mx(x, x_scales, ld_x_scales, w, w_scales, M, N, K, epi, out, out_scales,
                                      ld_out_scales, static_cast<float*>(ws), true, stream);
  if (epi == HR_EPI_RESIDUAL && ks > 1)
    hr::launch_residual_sum(static_cast<float*>(out), static_cast<const float*>(ws), ks, size_t(M) * size_t(N),
                            stream);
  return check_launch("linear mxfp4");
}

hr_status hr_qknorm_rope_kv(const hr_dims* dims, const hr_batch* batch, const void* qkv, const void* q_norm_w,
                            const void* k_norm_w, void* q_out, const hr_kv* kv, hipStream_t stream) {
  HR_TRY(check_dims(dims));
  HR_TRY(check_kv(dims, kv, "kv"));
  HR_TRY(check_batch(dims, batch, kv));
  HR_TRY(need(qkv, "qkv"));
  HR_TRY(need(q_norm_w, "q_norm_w"));
  HR_TRY(need(k_norm_w, "k_norm_w"));
  HR_TRY(need(q_out, "q_out"));
  if (batch->total_tokens == 0) return HR_OK;
  hr::launch_qknorm_rope_kv(qkv, batch->total_tokens, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                            dims->rope_theta, dims->rms_eps, batch->cu_seqlens, batch->start_pos,
                            batch->cache_slot, batch->used_keys, batch->n_seq, dims->causal != 0, q_norm_w,
                            k_norm_w, q_out, kv->k, kv->v, kv->capacity, stream);
  return check_launch("qknorm_rope_kv");
}

hr_status hr_attention(const hr_dims* dims, const hr_batch* batch, const void* q, const hr_kv* kv, void* out,
                       hr_wtype out_type, float out_scale, hipStream_t stream) {
  HR_TRY(check_dims(dims));
  HR_TRY(check_kv(dims, kv, "kv"));
  HR_TRY(check_batch(dims, batch, kv));
  HR_TRY(need(q, "q"));
  HR_TRY(need(out, "out"));
  if (out_type != HR_F16 && out_type != HR_FP8_E4M3) return fail(HR_EINVAL, "out_type: HR_F16 or HR_FP8_E4M3");
  if (out_type == HR_FP8_E4M3 && !(out_scale > 0.f)) return fail(HR_EINVAL, "out_scale must be > 0");
  if (batch->total_tokens == 0) return HR_OK;
  const hr::AttnSplit plan = attn_plan(dims, batch, nullptr);
  hr::launch_attention(q, kv->k, kv->v, batch->cu_seqlens, batch->start_pos, batch->cache_slot, batch->used_keys,
                       batch->n_seq, batch->max_seqlen, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                       kv->capacity, dims->causal != 0, out, out_type == HR_FP8_E4M3,
                       out_type == HR_FP8_E4M3 ? 1.0f / out_scale : 1.f, stream, &plan);
  return check_launch("attention");
}

hr_status hr_attention_f16(const hr_dims* dims, const hr_batch* batch, const void* q, const void* k16,
                           const void* v16, int32_t Tp, void* out, hr_wtype out_type, float out_scale,
                           hipStream_t stream) {
  HR_TRY(check_dims(dims));
  hr_kv unbounded{nullptr, nullptr, INT32_MAX, INT32_MAX};   // no cache: slots and capacity unchecked
  HR_TRY(check_batch(dims, batch, &unbounded));
  HR_TRY(need(q, "q"));
  HR_TRY(need(k16, "k16"));
  HR_TRY(need(v16, "v16"));
  HR_TRY(need(out, "out"));
  if (out_type != HR_F16 && out_type != HR_FP8_E4M3) return fail(HR_EINVAL, "out_type: HR_F16 or HR_FP8_E4M3");
  if (out_type == HR_FP8_E4M3 && !(out_scale > 0.f)) return fail(HR_EINVAL, "out_scale must be > 0");
  const int T = batch->total_tokens;
  if (Tp % 32 != 0 || Tp < (T + 31) / 32 * 32)
    return fail(HR_EINVAL, "Tp = %d: a multiple of 32 of at least %d", Tp, (T + 31) / 32 * 32);
  for (int s = 0; s < batch->n_seq; ++s) {
    if (batch->h_start_pos[s] != 0)
      return fail(HR_EUNSUPPORTED, "start_pos[%d] = %d: every sequence must start at position 0", s,
                  batch->h_start_pos[s]);
    if (batch->h_cu_seqlens[s] % 8 != 0)
      return fail(HR_EUNSUPPORTED, "cu_seqlens[%d] = %d is not a multiple of 8", s, batch->h_cu_seqlens[s]);
  }
  if (T == 0) return HR_OK;
  hr::launch_attention_f16(q, k16, v16, Tp, batch->cu_seqlens, batch->used_keys, batch->n_seq, batch->max_seqlen,
                           dims->n_q_heads, dims->n_kv_heads, dims->head_dim, dims->causal != 0, out,
                           out_type == HR_FP8_E4M3, out_type == HR_FP8_E4M3 ? 1.0f / out_scale : 1.f, stream);
  return check_launch("attention_f16");
}

hr_status hr_qknorm_rope_attention(const hr_dims* dims, const hr_batch* batch, const void* qkv,
                                   const void* q_norm_w, const void* k_norm_w, const hr_kv* kv, void* out,
                                   hr_wtype out_type, float out_scale, hipStream_t stream) {
  HR_TRY(check_dims(dims));
  HR_TRY(check_kv(dims, kv, "kv"));
  HR_TRY(check_batch(dims, batch, kv));
  HR_TRY(need(qkv, "qkv"));
  HR_TRY(need(q_norm_w, "q_norm_w"));
  HR_TRY(need(k_norm_w, "k_norm_w"));
  HR_TRY(need(out, "out"));
  if (out_type != HR_F16 && out_type != HR_FP8_E4M3) return fail(HR_EINVAL, "out_type: HR_F16 or HR_FP8_E4M3");
  if (out_type == HR_FP8_E4M3 && !(out_scale > 0.f)) return fail(HR_EINVAL, "out_scale must be > 0");
  const int longest = small_prompt(batch);
  if (longest < 0)
    return fail(HR_EUNSUPPORTED, "every sequence must start at position 0 with at most %d rows", hr::kSmallRows);
  if (batch->total_tokens == 0) return HR_OK;
  hr::launch_rope_attn_small(qkv, batch->n_seq, longest, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                             dims->rope_theta, dims->rms_eps, batch->cu_seqlens, batch->cache_slot,
                             batch->used_keys, dims->causal != 0, q_norm_w, k_norm_w, kv->k, kv->v, kv->capacity,
                             out, out_type == HR_FP8_E4M3, out_type == HR_FP8_E4M3 ? 1.0f / out_scale : 1.f,
                             stream);
  return check_launch("qknorm_rope_attention");
}

size_t hr_attention_chunked_workspace_bytes(const hr_dims* dims, int32_t total_tokens, int32_t n_slots) {
  if (!dims || total_tokens < 0 || n_slots < 1) return 0;
  const size_t t = size_t(total_tokens), S = size_t(n_slots), Hq = size_t(dims->n_q_heads);
  return up256(S * t * Hq * size_t(dims->head_dim) * 4) + up256(S * t * Hq * 8);
}

hr_status hr_attention_chunked(const hr_dims* dims, const hr_batch* batch, const void* q, const hr_kv* kv,
                               void* out, hr_wtype out_type, float out_scale, int32_t chunk_tiles,
                               int32_t n_slots, void* ws, size_t ws_bytes, hipStream_t stream) {
  HR_TRY(check_dims(dims));
  HR_TRY(check_kv(dims, kv, "kv"));
  HR_TRY(check_batch(dims, batch, kv));
  HR_TRY(need(q, "q"));
  HR_TRY(need(out, "out"));
  if (out_type != HR_F16 && out_type != HR_FP8_E4M3) return fail(HR_EINVAL, "out_type: HR_F16 or HR_FP8_E4M3");
  if (out_type == HR_FP8_E4M3 && !(out_scale > 0.f)) return fail(HR_EINVAL, "out_scale must be > 0");
  if (chunk_tiles < 1 || n_slots < 1 || n_slots > 64)
    return fail(HR_EINVAL, "chunk_tiles must be >= 1 and n_slots in [1, 64] (got %d, %d)", chunk_tiles, n_slots);
  if (batch->total_tokens == 0) return HR_OK;
  const size_t need_ws = hr_attention_chunked_workspace_bytes(dims, batch->total_tokens, n_slots);
  if (!ws || ws_bytes < need_ws)
    return fail(HR_EWORKSPACE, "attention workspace needs %zu bytes, got %zu", need_ws, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(HR_EALIGN, "workspace must be 256-byte aligned");
  const size_t t = size_t(batch->total_tokens), Hq = size_t(dims->n_q_heads);
  hr::AttnSplit sp;
  sp.decode = one_row_batch(batch);
  sp.chunk_tiles = chunk_tiles;
  sp.n_slots = n_slots;
  sp.part_o = static_cast<float*>(ws);
  sp.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + up256(size_t(n_slots) * t * Hq * dims->head_dim * 4));
  sp.T = batch->total_tokens;
  hr::launch_attention(q, kv->k, kv->v, batch->cu_seqlens, batch->start_pos, batch->cache_slot, batch->used_keys,
                       batch->n_seq, batch->max_seqlen, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                       kv->capacity, dims->causal != 0, out, out_type == HR_FP8_E4M3,
                       out_type == HR_FP8_E4M3 ? 1.0f / out_scale : 1.f, stream, &sp);
  return check_launch("attention (key chunks)");
}

size_t hr_head_workspace_bytes(int32_t n_seq, int32_t D) {
  (void)n_seq;
  return D > 0 ? up256(size_t(64) * D * 2) : 0;
}

hr_status hr_head_logits(const float* h, const hr_batch* batch, int32_t D, const void* final_norm_w, float eps,
                         const void* head_w, int32_t n_codebooks, int32_t cb_vocab, float* logits_out, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (!batch || batch->n_seq <= 0 || !batch->cu_seqlens || !batch->h_cu_seqlens)
    return fail(HR_EINVAL, "batch with n_seq > 0 and cu_seqlens required");
  if (D <= 0 || D % 64 || D > 8192) return fail(HR_EUNSUPPORTED, "D = %d must be a positive multiple of 64", D);
  if (n_codebooks <= 0 || cb_vocab <= 0) return fail(HR_EINVAL, "n_codebooks and cb_vocab must be > 0");
  for (int s = 0; s < batch->n_seq; ++s)
    if (batch->h_cu_seqlens[s + 1] <= batch->h_cu_seqlens[s])
      return fail(HR_EINVAL, "sequence %d is empty: no last row for the head", s);
  HR_TRY(need(h, "h"));
  HR_TRY(need(final_norm_w, "final_norm_w"));
  HR_TRY(need(head_w, "head_w"));
  HR_TRY(need(logits_out, "logits_out"));
  HR_TRY(need(ws, "ws"));
  if (ws_bytes < hr_head_workspace_bytes(batch->n_seq, D)) return fail(HR_EWORKSPACE, "head workspace too small");
  return run_head(h, batch, D, final_norm_w, eps, head_w, n_codebooks, cb_vocab, logits_out, ws, stream);
}

hr_status hr_quantize_weight_e4m3(const void* w, int32_t N, int32_t K, uint8_t* w8, float* scale,
                                  hipStream_t stream) {
  if (N <= 0 || K <= 0) return fail(HR_EINVAL, "bad N=%d K=%d", N, K);
  if (!w || !w8 || !scale) return fail(HR_EINVAL, "NULL pointer");
  hr::launch_quant_weight(w, N, K, w8, scale, stream);
  return check_launch("quantize_weight");
}

}  // extern "C"
