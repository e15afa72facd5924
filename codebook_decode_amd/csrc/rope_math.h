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
__device__ __forceinline__ float h_at(const u32x4& v, int i) {    // fp16 element i < 8 (i constant)
  return (i & 1) ? h_hi(v[i >> 1]) : h_lo(v[i >> 1]);
}

// 8 consecutive fp32 values of a head row (two 16-byte loads)
struct F8 {
  floatx4 a, b;
  __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};
__device__ __forceinline__ F8 load_f8(const float* p) {
  return F8{reinterpret_cast<const floatx4*>(p)[0], reinterpret_cast<const floatx4*>(p)[1]};
}
__device__ __forceinline__ u32x4 pack8_bf16(const F8& v) {      // nearest even (the cache format)
  return u32x4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])};
}
__device__ __forceinline__ u32x4 pack8_f16(const F8& v) {       // nearest even (q for the attention)
  return u32x4{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7])};
}

// The arithmetic below is spelled out operation by operation (explicit fmaf,
// no contraction): these helpers are inlined into several kernels, and a
// compiler free to fuse a multiply into an add could fuse them differently in
// each, so the cache rows and q would differ between paths in the last bit.

// sum of squares of a lane's 8 pairs of a head row
__device__ __forceinline__ float pairs_sumsq(const F8& lo, const F8& hi) {
#pragma clang fp contract(off)
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ss = __builtin_fmaf(lo[i], lo[i], ss);
    ss = __builtin_fmaf(hi[i], hi[i], ss);
  }
  return ss;
}

// a lane's 8 RoPE pairs (m, m + d/2), m = 8c + i, of an fp32 head row: RMSNorm
// scale inv and bf16 norm weights (w0: first half, w1: second half), then the
// rotation by the angles cs[i], sn[i]; fp32 results (the caller rounds them
// once, to bf16 for the cache or fp16 for q)
__device__ __forceinline__ void rope_pairs(const F8& lo, const F8& hi, const u32x4& w0, const u32x4& w1,
                                           float inv, const float* cs, const float* sn, F8& o0, F8& o1) {
#pragma clang fp contract(off)
  float y0[8], y1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = (lo[i] * inv) * bf_at(w0, i);
    const float b = (hi[i] * inv) * bf_at(w1, i);
    const float c = cs[i], s = sn[i];
    y0[i] = __builtin_fmaf(a, c, -(b * s));
    y1[i] = __builtin_fmaf(b, c, a * s);
  }
  o0 = F8{floatx4{y0[0], y0[1], y0[2], y0[3]}, floatx4{y0[4], y0[5], y0[6], y0[7]}};
  o1 = F8{floatx4{y1[0], y1[1], y1[2], y1[3]}, floatx4{y1[4], y1[5], y1[6], y1[7]}};
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
