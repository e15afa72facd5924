// Fused per-head q/k RMSNorm + rotate-half RoPE + KV-cache write (step A3).
// Sources: "Stabilize Higgs Audio termination and prefill", Summary (q/k norm +
// RoPE and KV writes kernelised in the batched prefill); flashrt-structures
// prefill_tower/fp8_chain.py `_build_rope` (rotate-half: the cosine table is
// the same over both halves of head_dim, so pair (m, m + d/2) turns together)
// and `run` (split the merged QKV rows, rotate, write the cache).
//
// A workgroup of 256 threads takes tpb <= kRopeTok tokens (1 for small
// batches, so the rows of a 13-token prompt spread over 13 workgroups).  First the per-token angle
// tables: p * theta^(-2m/d) for m < d/2, the frequency and the angle in
// float64, reduced to [-pi, pi] in float64, its sine and cosine taken in fp32,
// kept in LDS.  Then every head row of those tokens is handled by d/16 lanes, lane c
// owning the 8 RoPE pairs (8c + i, d/2 + 8c + i), i < 8: it reads the two
// 16-byte halves straight from the merged QKV row (the d/16 lanes of a row
// read 2 x d bytes, whole 128-byte lines), the head's sum of squares is a
// butterfly over those lanes, and the results leave as 16-byte stores.  Rows
// are dealt to the threads in rounds of 256 / (d/16), kRopeRows rounds in flight.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace hr {

constexpr int kRopeTok = 4;     // tokens per workgroup
constexpr int kRopeRows = 3;    // head-row rounds with loads in flight per thread

__device__ __forceinline__ float bf_at(const u32x4& v, int i) {   // element i < 8 (i constant)
  return (i & 1) ? bf_hi(v[i >> 1]) : bf_lo(v[i >> 1]);
}

// theta^(-2m/d), m < d/2, in float64: computed once on the host per launch and
// passed by value (kernel-argument memory), so no workgroup spends time on it
struct RopeFreq {
  double inv[64];
};

static RopeFreq rope_freq(int d, float theta) {
  RopeFreq f{};
  for (int m = 0; m < d / 2 && m < 64; ++m)
    f.inv[m] = std::exp2(-double(2 * m) / double(d) * std::log2(double(theta)));
  return f;
}

__global__ __launch_bounds__(256) void qknorm_rope_kv_kernel(
    const uint16_t* __restrict__ qkv, int T, int tpb, int Hq, int Hkv, int d, const RopeFreq freq, float eps,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ cache_slot, const int32_t* __restrict__ used_keys, int n_seq,
    int causal, const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
    uint16_t* __restrict__ q_out, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    int capacity) {
  __shared__ float s_cos[kRopeTok][64], s_sin[kRopeTok][64];
  __shared__ long long s_crow[kRopeTok];     // cache row (slot * capacity + position)
  __shared__ int s_wkv[kRopeTok];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * tpb;
  const int nt = min(tpb, T - t0);
  const int half = d >> 1;
  const int n_rows = Hq + 2 * Hkv;

  const int L = d >> 4;                       // lanes per head row
  const int c = tid % L;                      // this lane's 8-pair chunk
  const int per_round = 256 / L;
  const int total = nt * n_rows;
  const int step = per_round * kRopeRows;

  // head rows of one round of kRopeRows x per_round rows
  u32x4 lo[kRopeRows], hi[kRopeRows];
  auto load_round = [&](int base) {
#pragma unroll
    for (int k = 0; k < kRopeRows; ++k) {
      const int rr = base + k * per_round;
      if (rr < total) {
        const int tt = rr / n_rows, r = rr % n_rows;
        const uint16_t* src = qkv + size_t(t0 + tt) * n_rows * d + size_t(r) * d;
        lo[k] = *reinterpret_cast<const u32x4*>(src + 8 * c);
        hi[k] = *reinterpret_cast<const u32x4*>(src + half + 8 * c);
      } else {
        lo[k] = u32x4{0u, 0u, 0u, 0u};
        hi[k] = lo[k];
      }
    }
  };
  // the first round's rows and this lane's norm weights are requested before
  // the tables are built, so their latency overlaps the tables'
  int base = tid / L;
  load_round(base);
  const u32x4 wq0 = *reinterpret_cast<const u32x4*>(qw + 8 * c);
  const u32x4 wq1 = *reinterpret_cast<const u32x4*>(qw + half + 8 * c);
  const u32x4 wk0 = *reinterpret_cast<const u32x4*>(kw + 8 * c);
  const u32x4 wk1 = *reinterpret_cast<const u32x4*>(kw + half + 8 * c);

  // token positions, cache rows, whether K/V are written
  if (tid < nt) {
    const int t = t0 + tid;
    const int s = find_seq(cu, n_seq, t);
    const int i = t - cu[s];
    const int p = start_pos[s] + i;
    s_crow[tid] = (long long)cache_slot[s] * capacity + p;
    s_wkv[tid] = (causal || i < used_keys[s]) ? 1 : 0;
  }
  // angle tables: thread -> (token, m)
  for (int a = tid; a < nt * half; a += 256) {
    const int tt = a / half, m = a % half;
    const int t = t0 + tt;
    const int s = find_seq(cu, n_seq, t);
    const int p = start_pos[s] + (t - cu[s]);
    const double phi = double(p) * freq.inv[m];
    const double k2 = __builtin_rint(phi * 0.15915494309189535);
    const float red = float(__builtin_fma(-k2, 6.283185307179586, phi));
    float sn, cs;
    sincosf(red, &sn, &cs);
    s_cos[tt][m] = cs;
    s_sin[tt][m] = sn;
  }
  __syncthreads();

  for (; base < total; base += step) {
    if (base != tid / L) load_round(base);
#pragma unroll
    for (int k = 0; k < kRopeRows; ++k) {
      const int rr = base + k * per_round;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = bf_at(lo[k], i), b = bf_at(hi[k], i);
        ss += a * a + b * b;
      }
      ss = group_sum(ss, L);                  // every lane of the wave takes part
      if (rr >= total) continue;
      const int tt = rr / n_rows, r = rr % n_rows;
      const int t = t0 + tt;
      if (r < Hq + Hkv) {
        const bool is_q = r < Hq;
        if (!is_q && !s_wkv[tt]) continue;
        const float inv = 1.0f / __builtin_sqrtf(ss / float(d) + eps);
        u32x4 o0, o1;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          float y0[2], y1[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int m = 8 * c + i + e;
            const float a = bf_at(lo[k], i + e) * inv * bf_at(is_q ? wq0 : wk0, i + e);
            const float b = bf_at(hi[k], i + e) * inv * bf_at(is_q ? wq1 : wk1, i + e);
            const float cs = s_cos[tt][m], sn = s_sin[tt][m];
            y0[e] = a * cs - b * sn;
            y1[e] = b * cs + a * sn;
          }
          o0[i / 2] = pack_bf2(y0[0], y0[1]);
          o1[i / 2] = pack_bf2(y1[0], y1[1]);
        }
        uint16_t* dst = is_q ? q_out + (size_t(t) * Hq + r) * d
                             : kc + (size_t(s_crow[tt]) * Hkv + (r - Hq)) * d;
        *reinterpret_cast<u32x4*>(dst + 8 * c) = o0;
        *reinterpret_cast<u32x4*>(dst + half + 8 * c) = o1;
      } else if (s_wkv[tt]) {
        uint16_t* dst = vc + (size_t(s_crow[tt]) * Hkv + (r - Hq - Hkv)) * d;
        *reinterpret_cast<u32x4*>(dst + 8 * c) = lo[k];
        *reinterpret_cast<u32x4*>(dst + half + 8 * c) = hi[k];
      }
    }
  }
}

void launch_qknorm_rope_kv(const void* qkv, int T, int Hq, int Hkv, int d, float theta, float eps,
                           const int32_t* cu, const int32_t* start_pos, const int32_t* cache_slot,
                           const int32_t* used_keys, int n_seq, bool causal, const void* qw,
                           const void* kw, void* q_out, void* kc, void* vc, int capacity,
                           hipStream_t st) {
  // tokens per workgroup: 1 below 512 tokens (latency: every row in flight
  // at once), up to kRopeTok for large batches (fewer angle tables)
  const int tpb = T < 512 ? 1 : (T < 1024 ? 2 : kRopeTok);
  const int blocks = (T + tpb - 1) / tpb;
  const RopeFreq freq = rope_freq(d, theta);
  qknorm_rope_kv_kernel<<<blocks, 256, 0, st>>>(
      static_cast<const uint16_t*>(qkv), T, tpb, Hq, Hkv, d, freq, eps, cu, start_pos, cache_slot,
      used_keys, n_seq, causal ? 1 : 0, static_cast<const uint16_t*>(qw),
      static_cast<const uint16_t*>(kw), static_cast<uint16_t*>(q_out), static_cast<uint16_t*>(kc),
      static_cast<uint16_t*>(vc), capacity);
}

}  // namespace hr
