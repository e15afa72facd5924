// Fused per-head q/k RMSNorm + rotate-half RoPE + KV-cache write (step A3).
// Sources: "Stabilize Higgs Audio termination and prefill", Summary (q/k norm +
// RoPE and KV writes kernelised in the batched prefill); flashrt-structures
// prefill_tower/fp8_chain.py `_build_rope` (rotate-half: the cosine table is
// the same over both halves of head_dim, so pair (m, m + d/2) turns together)
// and `run` (split the merged QKV rows, rotate, write the cache).
//
// One workgroup per token.  The token's merged QKV row is staged in LDS with
// 128-bit loads issued together (so the per-head loop makes no global round
// trips); the d/2 angles p * theta^(-2m/d) are computed once per token in
// float64 (sincos of the double angle, rounded to fp32) and kept in LDS.  A
// head row of d values is handled by d/2 lanes, lane m owning the RoPE pair
// (m, m + d/2), so the rotation needs no lane exchange and the head's sum of
// squares is a butterfly over d/2 lanes.
#include "common.h"
#include "launch.h"

namespace hr {

__global__ __launch_bounds__(256) void qknorm_rope_kv_kernel(
    const uint16_t* __restrict__ qkv, int Hq, int Hkv, int d, float theta, float eps,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ cache_slot, const int32_t* __restrict__ used_keys, int n_seq,
    int causal, const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
    uint16_t* __restrict__ q_out, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    int capacity) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_row[];   // the token's qkv row
  __shared__ float s_cos[64], s_sin[64];
  const int t = blockIdx.x;
  const int n_rows = Hq + 2 * Hkv;
  const int qkv_w = n_rows * d;
  // stage the whole row with 128-bit loads (all issued before any use)
  const u32x4* src = reinterpret_cast<const u32x4*>(qkv + size_t(t) * qkv_w);
  for (int c = threadIdx.x; c < (qkv_w >> 3); c += blockDim.x)
    reinterpret_cast<u32x4*>(s_row)[c] = src[c];
  const int s = find_seq(cu, n_seq, t);
  const int i = t - cu[s];
  const int p = start_pos[s] + i;
  const bool write_kv = causal || i < used_keys[s];
  const size_t row = size_t(cache_slot[s]) * capacity + p;
  const int half = d >> 1;
  if (threadIdx.x < half) {
    double inv = exp2(-double(2 * threadIdx.x) / double(d) * log2(double(theta)));
    double phi = double(p) * inv;
    double sn, cs;
    sincos(phi, &sn, &cs);
    s_cos[threadIdx.x] = float(cs);
    s_sin[threadIdx.x] = float(sn);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per_wave = 64 / half;                 // head rows per wavefront pass
  const int sub = lane / half, m = lane % half;
  const float c = s_cos[m], sn = s_sin[m];
  const float wq0 = bf2f(qw[m]), wq1 = bf2f(qw[m + half]);
  const float wk0 = bf2f(kw[m]), wk1 = bf2f(kw[m + half]);
  for (int r0 = wave * per_wave; r0 < n_rows; r0 += 4 * per_wave) {
    const int r = r0 + sub;
    const bool valid = r < n_rows;
    float x0 = 0.f, x1 = 0.f;
    if (valid) { x0 = bf2f(s_row[r * d + m]); x1 = bf2f(s_row[r * d + m + half]); }
    float ss = group_sum(x0 * x0 + x1 * x1, half);
    if (!valid) continue;
    if (r < Hq + Hkv) {
      const bool is_q = r < Hq;
      const float inv = 1.0f / __builtin_sqrtf(ss / float(d) + eps);
      const float a = x0 * inv * (is_q ? wq0 : wk0);
      const float b = x1 * inv * (is_q ? wq1 : wk1);
      const float y0 = a * c - b * sn;
      const float y1 = b * c + a * sn;
      uint16_t* dst = is_q ? q_out + (size_t(t) * Hq + r) * d
                           : kc + (row * Hkv + (r - Hq)) * d;
      if (is_q || write_kv) { dst[m] = uint16_t(f2bf(y0)); dst[m + half] = uint16_t(f2bf(y1)); }
    } else if (write_kv) {
      uint16_t* dst = vc + (row * Hkv + (r - Hq - Hkv)) * d;
      dst[m] = s_row[r * d + m];
      dst[m + half] = s_row[r * d + m + half];
    }
  }
}

void launch_qknorm_rope_kv(const void* qkv, int T, int Hq, int Hkv, int d, float theta, float eps,
                           const int32_t* cu, const int32_t* start_pos, const int32_t* cache_slot,
                           const int32_t* used_keys, int n_seq, bool causal, const void* qw,
                           const void* kw, void* q_out, void* kc, void* vc, int capacity,
                           hipStream_t st) {
  const size_t shm = size_t(Hq + 2 * Hkv) * d * sizeof(uint16_t);
  qknorm_rope_kv_kernel<<<T, 256, shm, st>>>(
      static_cast<const uint16_t*>(qkv), Hq, Hkv, d, theta, eps, cu, start_pos, cache_slot,
      used_keys, n_seq, causal ? 1 : 0, static_cast<const uint16_t*>(qw),
      static_cast<const uint16_t*>(kw), static_cast<uint16_t*>(q_out), static_cast<uint16_t*>(kc),
      static_cast<uint16_t*>(vc), capacity);
}

}  // namespace hr
