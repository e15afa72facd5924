// Per-row q/k RMSNorm + rotate-half RoPE arithmetic shared by the kernels that
// apply it (step A3 alone, fused with the short-prompt attention, fused with
// the decode attention), so every path writes the same bits to the KV cache.
// Sources: "Stabilize Higgs Audio termination and prefill", Summary (q/k norm +
// RoPE kernelised); flashrt-structures prefill_tower/fp8_chain.py `_build_rope`
// (rotate-half: pair (m, m + d/2) turns by one angle).
#pragma once
#include <cmath>

#include "common.h"

namespace hr {

__device__ __forceinline__ float bf_at(const u32x4& v, int i) {   // element i < 8 (i constant)
  return (i & 1) ? bf_hi(v[i >> 1]) : bf_lo(v[i >> 1]);
}

// sum of squares of a lane's 8 pairs of a head row
__device__ __forceinline__ float pairs_sumsq(const u32x4& lo, const u32x4& hi) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = bf_at(lo, i), b = bf_at(hi, i);
    ss += a * a + b * b;
  }
  return ss;
}

// a lane's 8 RoPE pairs (m, m + d/2), m = 8c + i: RMSNorm scale inv and norm
// weights (w0: first half, w1: second half), then the rotation by the angles
// cs[i], sn[i]; bf16 results
__device__ __forceinline__ void rope_pairs(const u32x4& lo, const u32x4& hi, const u32x4& w0, const u32x4& w1,
                                           float inv, const float* cs, const float* sn, u32x4& o0, u32x4& o1) {
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    float y0[2], y1[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float a = bf_at(lo, i + e) * inv * bf_at(w0, i + e);
      const float b = bf_at(hi, i + e) * inv * bf_at(w1, i + e);
      const float c = cs[i + e], s = sn[i + e];
      y0[e] = a * c - b * s;
      y1[e] = b * c + a * s;
    }
    o0[i / 2] = pack_bf2(y0[0], y0[1]);
    o1[i / 2] = pack_bf2(y1[0], y1[1]);
  }
}

// angle of pair m at position p: p * theta^(-2m/d) in float64, reduced to
// [-pi, pi] in float64, sine and cosine in fp32
__device__ __forceinline__ void rope_angle(int p, double inv_freq, float& cs, float& sn) {
  const double phi = double(p) * inv_freq;
  const double k2 = __builtin_rint(phi * 0.15915494309189535);
  const float red = float(__builtin_fma(-k2, 6.283185307179586, phi));
  sincosf(red, &sn, &cs);
}

// theta^(-2m/d), m < d/2, in float64: computed once on the host per launch and
// passed by value (kernel-argument memory), so no workgroup spends time on it
struct RopeFreq {
  double inv[64];
};

inline RopeFreq rope_freq(int d, float theta) {
  RopeFreq f{};
  for (int m = 0; m < d / 2 && m < 64; ++m)
    f.inv[m] = std::exp2(-double(2 * m) / double(d) * std::log2(double(theta)));
  return f;
}

}  // namespace hr
