// Device-side helpers shared by the gfx950 kernels: number formats, vector
// types for the MFMA builtins, wavefront (64-lane) reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hr {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

// the same rounding (nearest even) with gfx950's packed convert, one
// v_cvt_pk_bf16_f32 for two values; for hot loops on finite data
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2_hw(float lo, float hi) {
  float2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// ---------------------------------------------------------------- IEEE binary16
// Activations of the bf16-weight band are fp16 (11-bit significand): 8x less
// rounding error than bf16 at the same MFMA rate.  bf16 weights enter the fp16
// MFMAs converted in registers; that conversion is exact for every bf16 value
// of magnitude in [2^-17, 2^16) (fp16 keeps all 8 significand bits there, down
// to its subnormals); smaller ones round to the nearest multiple of 2^-24, and
// 2^16 or more would overflow (outside the weights this band accepts).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float h_lo(uint32_t w) { return float(__builtin_bit_cast(f16x2_t, w)[0]); }
__device__ __forceinline__ float h_hi(uint32_t w) { return float(__builtin_bit_cast(f16x2_t, w)[1]); }
// two fp32 -> packed fp16, nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  f2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}
__device__ __forceinline__ uint32_t f2h(float f) {        // one fp32 -> fp16 bits, nearest even
  return uint32_t(__builtin_bit_cast(uint16_t, _Float16(f)));
}
// 8 bf16 -> 8 fp16 (3 VALU per pair: two widenings by bit shift, one packed convert)
__device__ __forceinline__ uint32_t bf2_to_f16x2(uint32_t w) {
  return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
}
__device__ __forceinline__ u32x4 bf8_to_f16x8(u32x4 v) {
  return u32x4{bf2_to_f16x2(v[0]), bf2_to_f16x2(v[1]), bf2_to_f16x2(v[2]), bf2_to_f16x2(v[3])};
}

// ---------------------------------------------------------------- OCP E4M3
// fp32 -> e4m3fn code: nearest even, magnitudes beyond 448 saturate to 448.
// Normal E4M3 values are (1 + m/8) 2^(e-7), e in 1..15; subnormals m 2^-9.
__device__ __forceinline__ uint32_t f2e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;                    // NaN
  float af = __uint_as_float(a);
  uint32_t code;
  if (af >= 448.0f) {
    code = 0x7Eu;
  } else if (af < 0.015625f) {                           // below 2^-6: step 2^-9
    code = uint32_t(__builtin_rintf(af * 512.0f));       // 0..8; 8 is 2^-6 (code 8)
  } else {
    int e = int(a >> 23) - 127;                          // -6 .. 8
    uint32_t mant = a & 0x7FFFFFu;
    uint32_t keep = mant >> 20;
    uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep++;
    if (keep == 8u) { keep = 0; e++; }
    code = (uint32_t(e + 7) << 3) | keep;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code == 0 ? 0u : (code | sign);
}

__device__ __forceinline__ float e4m3_to_f(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------- MXFP4 (OCP MX)
// Shared exponent of a 32-element block with the given max |v|: floor(log2
// amax) - 2 (2 = the exponent of E2M1's largest value 6), clamped to
// [-127, 127]; -127 for a zero (or subnormal) amax.  The scale byte is e + 127.
__device__ __forceinline__ int mx_block_exp(float amax) {
  const int ex = int((__float_as_uint(amax) >> 23) & 0xFFu);
  if (ex == 0) return -127;
  const int e = ex - 127 - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// E2M1 code of y (nearest, ties to the even code, saturating at 6): the
// midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 between the magnitudes
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 go to codes 0, 2, 2, 4, 4, 6, 6
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
             : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  if (c != 0u && (__float_as_uint(y) >> 31)) c |= 8u;
  return c;
}
// byte offset of block kb of row r in the slab-interleaved scale layout
// [K / 128][ld][4] (the 4 blocks of one 128-element K slab of a row together)
__device__ __forceinline__ size_t mx_scale_off(int r, int kb, int ld) {
  return (size_t(kb >> 2) * size_t(ld) + size_t(r)) * 4 + (kb & 3);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
// sum over groups of `width` consecutive lanes (width a power of two <= 64)
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = width >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seq, int t) {
  int lo = 0, hi = n_seq - 1;                            // largest s with cu[s] <= t
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace hr
