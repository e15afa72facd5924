// RMSNorm family (flashrt-structures prefill_tower/fp8_chain.py, `run`: norm
// before the merged QKV and gate/up GEMMs, final fp32 RMSNorm times the final
// weight; eps 1e-6):
//   embed_rmsnorm : h = widen(embed[id]) (or given bf16 rows); x = RMS(h) * w
//   rmsnorm       : x = RMS(h) * w from the fp32 residual
//   (x in fp16, the GEMM input of the bf16-weight band, or e4m3)
//   final_split   : z = RMS(h[last row of s]) * w in fp32, stored as two bf16
//                   terms hi = bf16(z), lo = bf16(z - hi) for the head GEMM
//   quant_weight  : per-output-channel E4M3 packing of a bf16 weight
//   MXFP4 (OCP MX: E2M1 values, one E8M0 scale per 32 consecutive K values):
//   quant_mx      : weight packing w' = (w * col) * row, or activation rows
//                   x' = x * col, one thread per 32-value block
//   rmsnorm_mx    : x = RMS(h) * w * col straight to MXFP4 (4 threads per block)
// The fp32 residual h is read once into registers (one row per workgroup,
// 8 elements per thread, 128-bit accesses); the row sum of squares is a
// wavefront butterfly plus a cross-wave LDS step.
#include "common.h"
#include "launch.h"

namespace hr {

constexpr int kNormThreads = 256;
constexpr int kNormMaxPerThread = 4;  // chunks of 8 -> D <= 256 * 32 = 8192

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Write 8 normalised values as fp16 (16 B) or e4m3 (8 B).
__device__ __forceinline__ void store_x8(void* x_out, size_t idx8, const float* y, bool fp8,
                                         float inv_scale) {
  if (fp8) {
    u32x2 o;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) w |= f2e4m3(y[4 * j + i] * inv_scale) << (8 * i);
      o[j] = w;
    }
    reinterpret_cast<u32x2*>(x_out)[idx8] = o;
  } else {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_f16x2(y[2 * j], y[2 * j + 1]);
    reinterpret_cast<u32x4*>(x_out)[idx8] = o;
  }
}

// mode 0: h given (fp32 rows); mode 1: rows from embed[ids]; mode 2: bf16 rows given
template <int MODE>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    const float* __restrict__ h_in, const int32_t* __restrict__ ids,
    const uint16_t* __restrict__ rows_bf16, float* __restrict__ h_out, int D,
    const uint16_t* __restrict__ w, float eps, void* __restrict__ x_out, int fp8, float inv_scale) {
  __shared__ float red[kNormThreads / 64];
  const int t = blockIdx.x;
  const int n8 = D >> 3;
  // the norm weights are requested first: they are not on the path that waits
  // for the row's sum of squares
  u32x4 wq[kNormMaxPerThread];
#pragma unroll
  for (int c = 0; c < kNormMaxPerThread; ++c) {
    const int i8 = threadIdx.x + c * kNormThreads;
    wq[c] = i8 < n8 ? reinterpret_cast<const u32x4*>(w)[i8] : u32x4{0u, 0u, 0u, 0u};
  }
  float v[kNormMaxPerThread][8];
  float ss = 0.f;
  const uint16_t* src16 = nullptr;
  if (MODE == 1) src16 = rows_bf16 + size_t(ids[t]) * D;
  if (MODE == 2) src16 = rows_bf16 + size_t(t) * D;
#pragma unroll
  for (int c = 0; c < kNormMaxPerThread; ++c) {
    int i8 = threadIdx.x + c * kNormThreads;
    if (i8 < n8) {
      if (MODE == 0) {
        const floatx4* p = reinterpret_cast<const floatx4*>(h_in + size_t(t) * D) + 2 * i8;
        floatx4 a = p[0], b = p[1];
        v[c][0] = a[0]; v[c][1] = a[1]; v[c][2] = a[2]; v[c][3] = a[3];
        v[c][4] = b[0]; v[c][5] = b[1]; v[c][6] = b[2]; v[c][7] = b[3];
      } else {
        u32x4 q = reinterpret_cast<const u32x4*>(src16)[i8];
#pragma unroll
        for (int j = 0; j < 4; ++j) { v[c][2 * j] = bf_lo(q[j]); v[c][2 * j + 1] = bf_hi(q[j]); }
        floatx4* hp = reinterpret_cast<floatx4*>(h_out + size_t(t) * D) + 2 * i8;
        hp[0] = floatx4{v[c][0], v[c][1], v[c][2], v[c][3]};
        hp[1] = floatx4{v[c][4], v[c][5], v[c][6], v[c][7]};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += v[c][j] * v[c][j];
    }
  }
  float tot = block_sum(ss, red);
  float r = 1.0f / __builtin_sqrtf(tot / float(D) + eps);
#pragma unroll
  for (int c = 0; c < kNormMaxPerThread; ++c) {
    int i8 = threadIdx.x + c * kNormThreads;
    if (i8 < n8) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = v[c][2 * j] * r * bf_lo(wq[c][j]);
        y[2 * j + 1] = v[c][2 * j + 1] * r * bf_hi(wq[c][j]);
      }
      store_x8(x_out, size_t(t) * n8 + i8, y, fp8 != 0, inv_scale);
    }
  }
}

// Fused residual add + RMSNorm (steps A6, A9): h[t] += part[0][t] + ... +
// part[ks-1][t] (the split-K partials of the O or down projection, summed in
// split order, then added to h: a fixed order, so the result is the same on
// every run), then x = RMS(h[t]) * w in the OUT format: fp16, e4m3(x * inv),
// MXFP4 of x * col (OCP MX blocks of 32, the 4 threads of a block adjacent
// lanes), or nothing (the last layer's residual).  ks = 0: the plain RMSNorm
// of h.  One row per workgroup, 8 values per thread, 128-bit accesses.
template <int OUT, int CPT, int KB>
__global__ __launch_bounds__(kNormThreads) void residual_norm_kernel(
    float* __restrict__ h, const float* __restrict__ part, int ks, size_t part_stride, int D,
    const uint16_t* __restrict__ w, float eps, void* __restrict__ x_out, float inv_scale,
    const float* __restrict__ col, uint8_t* __restrict__ mx_scales, int mx_ld) {
  // CPT: chunks of 8 values per thread (D <= 2048 CPT)
  __shared__ float red[kNormThreads / 64];
  const int t = blockIdx.x;
  const int n8 = D >> 3;
  u32x4 wq[CPT];
  if constexpr (OUT != kNormNone) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int i8 = threadIdx.x + c * kNormThreads;
      wq[c] = i8 < n8 ? reinterpret_cast<const u32x4*>(w)[i8] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // h and every partial of the thread's chunks are requested before any sum
  // (KB partials per batch): the loads overlap instead of one memory round
  // trip per partial and chunk.  The sums keep the split order, h + (p0 + p1 + ...).
  floatx4 ha[CPT], hb[CPT], sa[CPT], sb[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int i8 = threadIdx.x + c * kNormThreads;
    if (i8 < n8) {
      const floatx4* hp = reinterpret_cast<const floatx4*>(h + size_t(t) * D) + 2 * i8;
      ha[c] = hp[0];
      hb[c] = hp[1];
    }
  }
  // KB = 6 is launched for ks <= 6 only: a single batch
  const int kz_end = KB == 6 ? min(ks, 1) : ks;
  for (int kz0 = 0; kz0 < kz_end; kz0 += KB) {
    floatx4 qa[KB][CPT], qb[KB][CPT];
#pragma unroll
    for (int u = 0; u < KB; ++u)
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int i8 = threadIdx.x + c * kNormThreads;
        if (kz0 + u < ks && i8 < n8) {
          const floatx4* q = reinterpret_cast<const floatx4*>(part + size_t(kz0 + u) * part_stride + size_t(t) * D) + 2 * i8;
          qa[u][c] = q[0];
          qb[u][c] = q[1];
        }
      }
#pragma unroll
    for (int u = 0; u < KB; ++u)
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        if (kz0 + u >= ks) continue;
        if (kz0 + u == 0) {
          sa[c] = qa[u][c];
          sb[c] = qb[u][c];
        } else {
          sa[c] += qa[u][c];
          sb[c] += qb[u][c];
        }
      }
  }
  float v[CPT][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int i8 = threadIdx.x + c * kNormThreads;
    if (i8 < n8) {
      floatx4 a = ha[c], b = hb[c];
      if (ks > 0) {
        a += sa[c];
        b += sb[c];
        floatx4* hp = reinterpret_cast<floatx4*>(h + size_t(t) * D) + 2 * i8;
        hp[0] = a;
        hp[1] = b;
      }
      v[c][0] = a[0]; v[c][1] = a[1]; v[c][2] = a[2]; v[c][3] = a[3];
      v[c][4] = b[0]; v[c][5] = b[1]; v[c][6] = b[2]; v[c][7] = b[3];
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += v[c][j] * v[c][j];
    }
  }
  if constexpr (OUT == kNormNone) return;
  const float tot = block_sum(ss, red);
  const float r = 1.0f / __builtin_sqrtf(tot / float(D) + eps);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int i8 = threadIdx.x + c * kNormThreads;
    if constexpr (OUT == kNormMX) {
      if (c * kNormThreads >= n8) break;            // uniform: every lane of a block takes part below
    }
    const bool ok = i8 < n8;
    float y[8];
    if (ok) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = v[c][2 * j] * r * bf_lo(wq[c][j]);
        y[2 * j + 1] = v[c][2 * j + 1] * r * bf_hi(wq[c][j]);
      }
    }
    if constexpr (OUT == kNormMX) {
      float am = 0.f;
      if (ok) {
        if (col) {
          const floatx4* c4 = reinterpret_cast<const floatx4*>(col + 8 * i8);   // 16-byte aligned (checked)
          const floatx4 c0 = c4[0], c1 = c4[1];
#pragma unroll
          for (int j = 0; j < 4; ++j) { y[j] = y[j] * c0[j]; y[4 + j] = y[4 + j] * c1[j]; }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(y[j]));
      }
      am = fmaxf(am, __shfl_xor(am, 1, kWave));
      am = fmaxf(am, __shfl_xor(am, 2, kWave));
      if (ok) {
        const int e = mx_block_exp(am);
        uint32_t wd = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) wd |= e2m1_code(ldexpf(y[j], -e)) << (4 * j);
        reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(x_out) + size_t(t) * (D / 2))[i8] = wd;
        if ((i8 & 3) == 0) mx_scales[mx_scale_off(t, i8 >> 2, mx_ld)] = uint8_t(e + 127);
      }
    } else {
      if (ok) store_x8(x_out, size_t(t) * n8 + i8, y, OUT == kNormE4M3, inv_scale);
    }
  }
}

// The residual add alone over a flat [n] array (n a multiple of 8): h[i] +=
// part[0][i] + ... + part[ks-1][i], the same order and operations as
// residual_norm_kernel, so both give the same bits.
__global__ __launch_bounds__(256) void residual_sum_kernel(float* __restrict__ h, const float* __restrict__ part,
                                                           int ks, size_t n) {
  const size_t n8 = n >> 3;
  for (size_t i8 = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i8 < n8; i8 += size_t(gridDim.x) * blockDim.x) {
    floatx4* hp = reinterpret_cast<floatx4*>(h) + 2 * i8;
    const floatx4 ha = hp[0], hb = hp[1];
    // all partials of a batch requested before the sums (split order kept)
    constexpr int KB = 4;
    floatx4 sa, sb;
    for (int kz0 = 0; kz0 < ks; kz0 += KB) {
      floatx4 qa[KB], qb[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u)
        if (kz0 + u < ks) {
          const floatx4* q = reinterpret_cast<const floatx4*>(part + size_t(kz0 + u) * n) + 2 * i8;
          qa[u] = q[0];
          qb[u] = q[1];
        }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        if (kz0 + u >= ks) continue;
        if (kz0 + u == 0) { sa = qa[u]; sb = qb[u]; }
        else { sa += qa[u]; sb += qb[u]; }
      }
    }
    hp[0] = ha + sa;
    hp[1] = hb + sb;
  }
}

void launch_residual_sum(float* h, const float* part, int ks, size_t n, hipStream_t st) {
  if (ks <= 0 || n == 0) return;
  const size_t n8 = n >> 3;
  const size_t blocks = (n8 + 255) / 256;
  residual_sum_kernel<<<unsigned(blocks < 4096 ? blocks : 4096), 256, 0, st>>>(h, part, ks, n);
}

void launch_residual_norm(float* h, const float* part, int ks, int T, int D, const void* w, float eps,
                          int out_mode, void* x_out, float inv_scale, const float* col, uint8_t* mx_scales,
                          int mx_ld, hipStream_t st) {
  const size_t stride = size_t(T) * size_t(D);
  const uint16_t* w16 = static_cast<const uint16_t*>(w);
  if (out_mode == kNormNone && ks <= 0) return;
  const int cpt = (D / 8 + kNormThreads - 1) / kNormThreads;   // 1 .. kNormMaxPerThread (D <= 8192)
  auto go = [&](auto kern) {
    kern<<<T, kNormThreads, 0, st>>>(h, part, ks, stride, D, w16, eps, x_out, inv_scale, col, mx_scales, mx_ld);
  };
  // partials per load batch: 4, or 6 for the five splits of the small-batch
  // residual projections at 2 chunks per thread (hidden sizes 2049-4096: one
  // round trip instead of two; the larger batch costs registers, so only there)
  const bool kb6 = cpt == 2 && ks > 4 && ks <= 6;
#define HR_NORM_CPT(MODE)                                                                   \
  switch (cpt) {                                                                            \
    case 1: go(residual_norm_kernel<MODE, 1, 4>); break;                                    \
    case 2: kb6 ? go(residual_norm_kernel<MODE, 2, 6>) : go(residual_norm_kernel<MODE, 2, 4>); break; \
    case 3: go(residual_norm_kernel<MODE, 3, 4>); break;                                    \
    default: go(residual_norm_kernel<MODE, 4, 4>);                                          \
  }
  switch (out_mode) {
    case kNormNone: HR_NORM_CPT(kNormNone); break;
    case kNormE4M3: HR_NORM_CPT(kNormE4M3); break;
    case kNormMX: HR_NORM_CPT(kNormMX); break;
    default: HR_NORM_CPT(kNormF16);
  }
#undef HR_NORM_CPT
}

// z = RMS(h[row]) * w (fp32); out rows s (hi) and n_rows + s (lo), bf16, stride D.
__global__ __launch_bounds__(kNormThreads) void final_split_kernel(
    const float* __restrict__ h, const int32_t* __restrict__ cu, int row0_seq, int D,
    const uint16_t* __restrict__ w, float eps, int n_rows, uint16_t* __restrict__ zsplit) {
  __shared__ float red[kNormThreads / 64];
  const int s = blockIdx.x;
  const int row = cu[row0_seq + s + 1] - 1;
  const int n8 = D >> 3;
  float v[kNormMaxPerThread][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kNormMaxPerThread; ++c) {
    int i8 = threadIdx.x + c * kNormThreads;
    if (i8 < n8) {
      const floatx4* p = reinterpret_cast<const floatx4*>(h + size_t(row) * D) + 2 * i8;
      floatx4 a = p[0], b = p[1];
      v[c][0] = a[0]; v[c][1] = a[1]; v[c][2] = a[2]; v[c][3] = a[3];
      v[c][4] = b[0]; v[c][5] = b[1]; v[c][6] = b[2]; v[c][7] = b[3];
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += v[c][j] * v[c][j];
    }
  }
  float tot = block_sum(ss, red);
  float r = 1.0f / __builtin_sqrtf(tot / float(D) + eps);
#pragma unroll
  for (int c = 0; c < kNormMaxPerThread; ++c) {
    int i8 = threadIdx.x + c * kNormThreads;
    if (i8 < n8) {
      u32x4 wq = reinterpret_cast<const u32x4*>(w)[i8];
      u32x4 hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float z0 = v[c][2 * j] * r * bf_lo(wq[j]);
        float z1 = v[c][2 * j + 1] * r * bf_hi(wq[j]);
        uint32_t h0 = f2bf(z0), h1 = f2bf(z1);
        hi[j] = h0 | (h1 << 16);
        lo[j] = pack_bf2(z0 - bf2f(uint16_t(h0)), z1 - bf2f(uint16_t(h1)));
      }
      reinterpret_cast<u32x4*>(zsplit + size_t(s) * D)[i8] = hi;
      reinterpret_cast<u32x4*>(zsplit + size_t(n_rows + s) * D)[i8] = lo;
    }
  }
}

// One workgroup per weight row: scale = max|w| / 448, codes = e4m3(w / scale).
__global__ __launch_bounds__(kNormThreads) void quant_weight_kernel(
    const uint16_t* __restrict__ w, int K, uint8_t* __restrict__ w8, float* __restrict__ scale) {
  __shared__ float red[kNormThreads / 64];
  const int n = blockIdx.x;
  const uint16_t* row = w + size_t(n) * K;
  float m = 0.f;
  for (int k = threadIdx.x; k < K; k += blockDim.x) m = fmaxf(m, fabsf(bf2f(row[k])));
  m = wave_max(m);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float amax = 0.f;
  for (int i = 0; i < int(blockDim.x >> 6); ++i) amax = fmaxf(amax, red[i]);
  float s = amax / 448.0f;
  if (!(s > 0.f)) s = 1.0f;
  if (threadIdx.x == 0) scale[n] = s;
  for (int k = threadIdx.x; k < K; k += blockDim.x) w8[size_t(n) * K + k] = uint8_t(f2e4m3(bf2f(row[k]) / s));
}

void launch_embed_rmsnorm(const int32_t* ids, const void* embed, const void* x_embeds, int T, int D,
                          const void* w, float eps, float* h_out, void* x_out, bool fp8,
                          float inv_scale, hipStream_t st) {
  const uint16_t* w16 = static_cast<const uint16_t*>(w);
  if (ids)
    rmsnorm_kernel<1><<<T, kNormThreads, 0, st>>>(nullptr, ids, static_cast<const uint16_t*>(embed),
                                                  h_out, D, w16, eps, x_out, fp8, inv_scale);
  else
    rmsnorm_kernel<2><<<T, kNormThreads, 0, st>>>(nullptr, nullptr,
                                                  static_cast<const uint16_t*>(x_embeds), h_out, D,
                                                  w16, eps, x_out, fp8, inv_scale);
}

void launch_rmsnorm(const float* h, int T, int D, const void* w, float eps, void* x_out, bool fp8,
                    float inv_scale, hipStream_t st) {
  // the fused kernel with no partials: the same arithmetic as after a residual add
  launch_residual_norm(const_cast<float*>(h), nullptr, 0, T, D, w, eps, fp8 ? kNormE4M3 : kNormF16, x_out, inv_scale,
                       nullptr, nullptr, 0, st);
}

void launch_final_split(const float* h, const int32_t* cu, int seq0, int n, int D, const void* w,
                        float eps, int n_rows, void* zsplit, hipStream_t st) {
  final_split_kernel<<<n, kNormThreads, 0, st>>>(h, cu, seq0, D, static_cast<const uint16_t*>(w),
                                                 eps, n_rows, static_cast<uint16_t*>(zsplit));
}

void launch_quant_weight(const void* w, int N, int K, uint8_t* w8, float* scale, hipStream_t st) {
  quant_weight_kernel<<<N, kNormThreads, 0, st>>>(static_cast<const uint16_t*>(w), K, w8, scale);
}

// ---------------------------------------------------------------- MXFP4
// Encode 32 values (one block) held by one thread: codes (16 B, element 2i in
// the low nibble of byte i) and the scale byte.
__device__ __forceinline__ void mx_encode32(const float* v, u32x4& codes, uint32_t& sbyte) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  const int e = mx_block_exp(am);
  sbyte = uint32_t(e + 127);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t wd = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) wd |= e2m1_code(ldexpf(v[8 * q + i], -e)) << (4 * i);
    codes[q] = wd;
  }
}

// One thread per (row, block).  SRC 0: bf16 rows, 1: fp32 rows, 2: fp16 rows.  v = x * col
// (one binary32 rounding) then * row (a second one), as the packing contract.
template <int SRC>
__global__ __launch_bounds__(256) void quant_mx_kernel(const void* __restrict__ x, int M, int K,
                                                       const float* __restrict__ col,
                                                       const float* __restrict__ row_scale,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                       int ld_s) {
  const int nb = K >> 5;
  const size_t id = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= size_t(M) * nb) return;
  const int r = int(id / nb), kb = int(id % nb);
  float v[32];
  if (SRC == 0) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + size_t(r) * K + kb * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 t = p[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) { v[8 * q + 2 * j] = bf_lo(t[j]); v[8 * q + 2 * j + 1] = bf_hi(t[j]); }
    }
  } else if (SRC == 2) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + size_t(r) * K + kb * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 t = p[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) { v[8 * q + 2 * j] = h_lo(t[j]); v[8 * q + 2 * j + 1] = h_hi(t[j]); }
    }
  } else {
    const floatx4* p = reinterpret_cast<const floatx4*>(static_cast<const float*>(x) + size_t(r) * K + kb * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const floatx4 t = p[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * q + j] = t[j];
    }
  }
  if (col) {
    const floatx4* c4 = reinterpret_cast<const floatx4*>(col + kb * 32);   // 16-byte aligned (checked)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const floatx4 c = c4[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * q + j] = v[4 * q + j] * c[j];
    }
  }
  if (row_scale) {
    const float rs = row_scale[r];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = v[i] * rs;
  }
  u32x4 c;
  uint32_t sb;
  mx_encode32(v, c, sb);
  reinterpret_cast<u32x4*>(codes + size_t(r) * (K / 2))[kb] = c;
  scales[mx_scale_off(r, kb, ld_s)] = uint8_t(sb);
}

void launch_quant_mx(const void* x, int fmt, int M, int K, const float* col, const float* row_scale,
                     uint8_t* codes, uint8_t* scales, int ld_s, hipStream_t st) {
  const size_t n = size_t(M) * (K / 32);
  const int grid = int((n + 255) / 256);
  if (fmt == 1) quant_mx_kernel<1><<<grid, 256, 0, st>>>(x, M, K, col, row_scale, codes, scales, ld_s);
  else if (fmt == 2) quant_mx_kernel<2><<<grid, 256, 0, st>>>(x, M, K, col, row_scale, codes, scales, ld_s);
  else quant_mx_kernel<0><<<grid, 256, 0, st>>>(x, M, K, col, row_scale, codes, scales, ld_s);
}

void launch_rmsnorm_mx(const float* h, int T, int D, const void* w, const float* col, float eps,
                       uint8_t* codes, uint8_t* scales, int ld_s, hipStream_t st) {
  launch_residual_norm(const_cast<float*>(h), nullptr, 0, T, D, w, eps, kNormMX, codes, 1.f, col, scales, ld_s, st);
}

}  // namespace hr
