// Projections of the prefill chain (steps A2 merged QKV, A5 output, A7 merged
// gate/up + SwiGLU, A8 down; A10 audio head) on gfx950 MFMA.
// Sources: flashrt-structures prefill_tower/fp8_chain.py (merged-QKV and merged
// gate/up GEMMs; FP8 GEMM alpha = activation scale x weight scale; the
// activation fused after the gate/up GEMM); "Stabilize Higgs Audio termination
// and prefill", Summary (projection GEMMs of the batched prefill).
//
// out = x [M, K] . W [N, K]^T, W row-major [out, in] as stored.
//
// Two kernels:
//  * skinny (M <= 64): weight streaming.  A workgroup owns 16 output columns
//    (16 gate + 16 up for SwiGLU) and its wavefronts split K; every lane streams
//    32 contiguous bytes of a weight row per step (16 rows x 128 B per wave, so
//    whole cache lines), the activation rows come from L2.  Cross-workgroup
//    split-K (grid.y) is allowed for the residual epilogue, reduced with fp32
//    atomics into h.  Wave partials are reduced in LDS in a fixed order.
//  * tiled (M > 64): 128 x 128 output tile per 256-thread workgroup, 2 x 2
//    wavefronts of 64 x 64 (4 x 4 MFMA 16x16 blocks), 128-byte K slabs double
//    buffered global -> registers -> LDS (rows padded by 16 B), one barrier
//    per slab.
// MFMA: v_mfma_f32_16x16x32_bf16 (8 bf16 per lane) or v_mfma_f32_16x16x32_fp8_fp8
// (8 e4m3 bytes per lane).  Lane l holds row/col l%16 and 8 consecutive k of
// lane group l/16; since A and B use the same k placement, any consistent
// assignment of memory k to (lane group, slot) is a valid contraction, which
// lets each lane read 16 contiguous bytes.  Accumulator: lane l has column
// l%16, rows 4*(l/16) + r.
#include "common.h"
#include "launch.h"

namespace hr {

__device__ __forceinline__ floatx4 mfma_bf16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_fp8(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                            floatx4 c) {
  long a = (long)(((unsigned long)a1 << 32) | a0);
  long b = (long)(((unsigned long)b1 << 32) | b0);
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}
// 16 bytes of A times 16 bytes of B along k: one bf16 MFMA or two fp8 MFMAs.
template <bool FP8>
__device__ __forceinline__ floatx4 mma16(u32x4 a, u32x4 b, floatx4 c) {
  if constexpr (FP8) {
    c = mfma_fp8(a[0], a[1], b[0], b[1], c);
    return mfma_fp8(a[2], a[3], b[2], b[3], c);
  } else {
    return mfma_bf16(a, b, c);
  }
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

struct EpiArgs {
  int epi;            // hr_epilogue
  void* out;          // bf16 [M,N] | fp32 [M,N] (+=) | act [M,F] | fp32 logits
  int ldo;            // leading dimension of out (elements)
  float x_scale;      // FP8: activation scale
  const float* w_scale;  // FP8: per-output-channel weight scale (N)
  float out_inv;      // SwiGLU FP8 output: 1 / activation scale of the next GEMM
  int out_fp8;        // SwiGLU output in e4m3
  int F;              // SwiGLU width (gate rows [0,F), up rows [F,2F))
  int hilo_rows;      // head: rows [0,h) hold hi, [h,2h) lo terms; out = hi + lo
};

// value of one product element after the dtype scale
template <bool FP8>
__device__ __forceinline__ float scaled(const EpiArgs& e, float acc, int n) {
  if constexpr (FP8) return acc * e.x_scale * e.w_scale[n];
  return acc;
}

// ============================================================== skinny kernel
template <int WAVES, int MB, int EPI, bool FP8>
__global__ __launch_bounds__(WAVES * 64) void gemm_skinny_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, int M, int N, int K_bytes,
    EpiArgs e) {
  constexpr int NB = (EPI == HR_EPI_SWIGLU) ? 2 : 1;   // gate and up column blocks
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cb = blockIdx.x;                           // 16-column block
  const int g = lane >> 4, rc = lane & 15;
  // weight rows this lane streams
  int wrow[NB];
  bool wok[NB];
  if constexpr (EPI == HR_EPI_SWIGLU) {
    wrow[0] = cb * 16 + rc;
    wrow[NB - 1] = e.F + cb * 16 + rc;
    wok[0] = true;
    wok[NB - 1] = true;
  } else {
    wrow[0] = cb * 16 + rc;
    wok[0] = wrow[0] < N;
  }
  const int steps = K_bytes >> 7;                      // 128-byte K steps
  const int ksplit = gridDim.y, kz = blockIdx.y;
  const int s_lo = (steps * kz) / ksplit, s_hi = (steps * (kz + 1)) / ksplit;

  floatx4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int U = 4;
  int s = s_lo + wave;
  for (; s + (U - 1) * WAVES < s_hi; s += U * WAVES) {
    u32x4 bw[U][NB][2], ax[U][MB][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t kb = size_t(s + u * WAVES) * 128 + g * 32;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4* p = reinterpret_cast<const u32x4*>(w + size_t(wrow[nb]) * K_bytes + kb);
        bw[u][nb][0] = wok[nb] ? p[0] : zero;
        bw[u][nb][1] = wok[nb] ? p[1] : zero;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = mb * 16 + rc;
        const u32x4* p = reinterpret_cast<const u32x4*>(x + size_t(row) * K_bytes + kb);
        ax[u][mb][0] = row < M ? p[0] : zero;
        ax[u][mb][1] = row < M ? p[1] : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[nb][mb] = mma16<FP8>(ax[u][mb][0], bw[u][nb][0], acc[nb][mb]);
          acc[nb][mb] = mma16<FP8>(ax[u][mb][1], bw[u][nb][1], acc[nb][mb]);
        }
  }
  for (; s < s_hi; s += WAVES) {
    const size_t kb = size_t(s) * 128 + g * 32;
    u32x4 bw[NB][2], ax[MB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const u32x4* p = reinterpret_cast<const u32x4*>(w + size_t(wrow[nb]) * K_bytes + kb);
      bw[nb][0] = wok[nb] ? p[0] : zero;
      bw[nb][1] = wok[nb] ? p[1] : zero;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = mb * 16 + rc;
      const u32x4* p = reinterpret_cast<const u32x4*>(x + size_t(row) * K_bytes + kb);
      ax[mb][0] = row < M ? p[0] : zero;
      ax[mb][1] = row < M ? p[1] : zero;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc[nb][mb] = mma16<FP8>(ax[mb][0], bw[nb][0], acc[nb][mb]);
        acc[nb][mb] = mma16<FP8>(ax[mb][1], bw[nb][1], acc[nb][mb]);
      }
  }

  // fixed-order reduction of the wavefront partials
  __shared__ floatx4 red[WAVES][NB][MB][64];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][nb][mb][lane] = acc[nb][mb];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MB * 64 * 4; idx += WAVES * 64) {
    const int r = idx & 3, ln = (idx >> 2) & 63, mb = idx >> 8;
    float v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float t = 0.f;
      for (int wv = 0; wv < WAVES; ++wv) t += red[wv][nb][mb][ln][r];
      v[nb] = t;
    }
    const int row = mb * 16 + 4 * (ln >> 4) + r;
    const int col = cb * 16 + (ln & 15);
    if constexpr (EPI == HR_EPI_SWIGLU) {
      if (row < M) {
        const float gt = scaled<FP8>(e, v[0], col);
        const float up = scaled<FP8>(e, v[NB - 1], e.F + col);
        const float a = silu(gt) * up;
        if (e.out_fp8)
          static_cast<uint8_t*>(e.out)[size_t(row) * e.ldo + col] = uint8_t(f2e4m3(a * e.out_inv));
        else
          static_cast<uint16_t*>(e.out)[size_t(row) * e.ldo + col] = uint16_t(f2bf(a));
      }
    } else if (col < N) {
      if constexpr (EPI == HR_EPI_BF16) {
        if (row < M)
          static_cast<uint16_t*>(e.out)[size_t(row) * e.ldo + col] =
              uint16_t(f2bf(scaled<FP8>(e, v[0], col)));
      } else if constexpr (EPI == HR_EPI_RESIDUAL) {
        if (row < M) {
          float* o = static_cast<float*>(e.out) + size_t(row) * e.ldo + col;
          if (ksplit == 1) *o += scaled<FP8>(e, v[0], col);
          else unsafeAtomicAdd(o, scaled<FP8>(e, v[0], col));
        }
      } else {  // HR_EPI_HEAD: fp32 logits = hi-row product + lo-row product
        if (row < e.hilo_rows) {
          const int r2 = row + e.hilo_rows;   // the lo term of the same sequence
          // r2 lives in the same workgroup (rows < 2*hilo_rows <= 64)
          float lo = 0.f;
          const int mb2 = r2 >> 4, q = r2 & 15;
          const int ln2 = (q >> 2) * 16 + (ln & 15), rr2 = q & 3;
          for (int wv = 0; wv < WAVES; ++wv) lo += red[wv][0][mb2 < MB ? mb2 : 0][ln2][rr2];
          static_cast<float*>(e.out)[size_t(row) * e.ldo + col] = v[0] + lo;
        }
      }
    }
  }
}

// ============================================================== tiled kernel
constexpr int TBM = 128, TBN = 128, TBK = 128;   // TBK in bytes
constexpr int TLD = TBK + 16;                    // padded LDS row (bytes)

template <int EPI, bool FP8>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(const uint8_t* __restrict__ x,
                                                         const uint8_t* __restrict__ w, int M, int N,
                                                         int K_bytes, int tiles_m, EpiArgs e) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* sA = smem;                       // [2][TBM][TLD]
  uint8_t* sB = smem + 2 * TBM * TLD;       // [2][TBN][TLD]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * TBM, n0 = tn * TBN;
  const int g = lane >> 4, rc = lane & 15;

  // global rows this thread copies (4 x 16 B of A and of B per slab)
  const uint8_t* ga[4];
  const uint8_t* gb[4];
  bool oka[4], okb[4];
  int lrow[4], lcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;
    lrow[j] = c >> 3;
    lcol[j] = (c & 7) * 16;
    const int ar = m0 + lrow[j];
    oka[j] = ar < M;
    ga[j] = x + size_t(oka[j] ? ar : 0) * K_bytes + lcol[j];
    int br;
    if constexpr (EPI == HR_EPI_SWIGLU) {
      const int blk = lrow[j] >> 4, off = lrow[j] & 15;
      const int a0 = (n0 >> 1) + (blk >> 1) * 16 + off;   // act column
      br = (blk & 1) ? e.F + a0 : a0;
      okb[j] = a0 < e.F;
    } else {
      br = n0 + lrow[j];
      okb[j] = br < N;
    }
    gb[j] = w + size_t(okb[j] ? br : 0) * K_bytes + lcol[j];
  }
  const int slabs_total = K_bytes / TBK;
  const int kz = blockIdx.z, ksplit = gridDim.z;
  const int sl0 = (slabs_total * kz) / ksplit, sl1 = (slabs_total * (kz + 1)) / ksplit;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[4], rb[4];
  auto gload = [&](int slab) {
    const size_t ko = size_t(slab) * TBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ra[j] = oka[j] ? *reinterpret_cast<const u32x4*>(ga[j] + ko) : zero;
      rb[j] = okb[j] ? *reinterpret_cast<const u32x4*>(gb[j] + ko) : zero;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4*>(sA + (buf * TBM + lrow[j]) * TLD + lcol[j]) = ra[j];
      *reinterpret_cast<u32x4*>(sB + (buf * TBN + lrow[j]) * TLD + lcol[j]) = rb[j];
    }
  };

  if (sl0 < sl1) {
    gload(sl0);
    sstore(0);
  }
  __syncthreads();
  int buf = 0;
  for (int sl = sl0; sl < sl1; ++sl) {
    const bool more = sl + 1 < sl1;
    if (more) gload(sl + 1);
    const uint8_t* A = sA + (buf * TBM + wm * 64) * TLD;
    const uint8_t* B = sB + (buf * TBN + wn * 64) * TLD;
#pragma unroll
    for (int ks = 0; ks < TBK; ks += 64) {           // 64-byte halves of the slab
      u32x4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(A + (i * 16 + rc) * TLD + ks + g * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(B + (j * 16 + rc) * TLD + ks + g * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma16<FP8>(fa[i], fb[j], acc[i][j]);
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // epilogue: lane holds column rc of each block, rows 4g + r
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * 64 + i * 16 + 4 * g + r;
      if (row >= M) continue;
      if constexpr (EPI == HR_EPI_SWIGLU) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int col = (n0 >> 1) + (wn * 2 + jj) * 16 + rc;
          if (col < e.F) {
            const float gt = scaled<FP8>(e, acc[i][2 * jj][r], col);
            const float up = scaled<FP8>(e, acc[i][2 * jj + 1][r], e.F + col);
            const float a = silu(gt) * up;
            if (e.out_fp8)
              static_cast<uint8_t*>(e.out)[size_t(row) * e.ldo + col] = uint8_t(f2e4m3(a * e.out_inv));
            else
              static_cast<uint16_t*>(e.out)[size_t(row) * e.ldo + col] = uint16_t(f2bf(a));
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn * 64 + j * 16 + rc;
          if (col >= N) continue;
          const float v = scaled<FP8>(e, acc[i][j][r], col);
          if constexpr (EPI == HR_EPI_BF16) {
            static_cast<uint16_t*>(e.out)[size_t(row) * e.ldo + col] = uint16_t(f2bf(v));
          } else {
            float* o = static_cast<float*>(e.out) + size_t(row) * e.ldo + col;
            if (ksplit == 1) *o += v; else unsafeAtomicAdd(o, v);
          }
        }
      }
    }
  }
}

// ============================================================== dispatch
template <int EPI, bool FP8>
static void skinny(const uint8_t* x, const uint8_t* w, int M, int N, int Kb, const EpiArgs& e,
                   int blocks, int ksplit, hipStream_t st) {
  dim3 grid(blocks, ksplit);
  const int mb = (M + 15) / 16;
  if (EPI == HR_EPI_SWIGLU) {
    if (mb == 1) gemm_skinny_kernel<8, 1, EPI, FP8><<<grid, 512, 0, st>>>(x, w, M, N, Kb, e);
    else if (mb == 2) gemm_skinny_kernel<4, 2, EPI, FP8><<<grid, 256, 0, st>>>(x, w, M, N, Kb, e);
    else gemm_skinny_kernel<4, 4, EPI, FP8><<<grid, 256, 0, st>>>(x, w, M, N, Kb, e);
  } else {
    if (mb == 1) gemm_skinny_kernel<8, 1, EPI, FP8><<<grid, 512, 0, st>>>(x, w, M, N, Kb, e);
    else if (mb == 2) gemm_skinny_kernel<8, 2, EPI, FP8><<<grid, 512, 0, st>>>(x, w, M, N, Kb, e);
    else gemm_skinny_kernel<4, 4, EPI, FP8><<<grid, 256, 0, st>>>(x, w, M, N, Kb, e);
  }
}

template <int EPI, bool FP8>
static void tiled(const uint8_t* x, const uint8_t* w, int M, int N, int Kb, const EpiArgs& e,
                  int ksplit, hipStream_t st) {
  const int tiles_m = (M + TBM - 1) / TBM;
  const int ncols = (EPI == HR_EPI_SWIGLU) ? 2 * e.F : N;
  const int tiles_n = (ncols + TBN - 1) / TBN;
  const size_t shm = size_t(2) * (TBM + TBN) * TLD;
  dim3 grid(tiles_m * tiles_n, 1, ksplit);
  static bool lds_raised = false;  // 72 KB of dynamic LDS: above the 64 KB default limit
  if (!lds_raised) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tiled_kernel<EPI, FP8>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, int(shm));
    lds_raised = true;
  }
  gemm_tiled_kernel<EPI, FP8><<<grid, 256, shm, st>>>(x, w, M, N, Kb, tiles_m, e);
}

void launch_linear(const void* x, const void* w, const float* w_scale, float x_scale, bool fp8,
                   int M, int N, int K, int epi, void* out, float out_scale, hipStream_t st) {
  EpiArgs e{};
  e.epi = epi;
  e.out = out;
  e.x_scale = x_scale;
  e.w_scale = w_scale;
  e.out_fp8 = (epi == HR_EPI_SWIGLU && fp8) ? 1 : 0;
  e.out_inv = out_scale > 0.f ? 1.0f / out_scale : 1.0f;
  e.F = N / 2;
  e.ldo = (epi == HR_EPI_SWIGLU) ? N / 2 : N;
  const int Kb = fp8 ? K : 2 * K;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  const int ncols = (epi == HR_EPI_SWIGLU) ? N / 2 : N;
  const int blocks = (ncols + 15) / 16;
#define HR_DISPATCH(EPI_)                                                                     \
  if (M <= 64) {                                                                              \
    int ks = 1;                                                                               \
    if (EPI_ == HR_EPI_RESIDUAL && blocks < 256) ks = (512 + blocks - 1) / blocks;            \
    if (ks > Kb / 128) ks = Kb / 128;                                                         \
    if (fp8) skinny<EPI_, true>(xb, wb, M, N, Kb, e, blocks, ks, st);                         \
    else skinny<EPI_, false>(xb, wb, M, N, Kb, e, blocks, ks, st);                            \
  } else {                                                                                    \
    const int tiles = ((M + TBM - 1) / TBM) * ((((EPI_ == HR_EPI_SWIGLU) ? N : N) + TBN - 1) / TBN); \
    int ks = 1;                                                                               \
    if (EPI_ == HR_EPI_RESIDUAL && tiles < 256) ks = (256 + tiles - 1) / tiles;               \
    if (ks > Kb / TBK) ks = Kb / TBK;                                                         \
    if (fp8) tiled<EPI_, true>(xb, wb, M, N, Kb, e, ks, st);                                  \
    else tiled<EPI_, false>(xb, wb, M, N, Kb, e, ks, st);                                     \
  }
  if (epi == HR_EPI_BF16) { HR_DISPATCH(HR_EPI_BF16) }
  else if (epi == HR_EPI_RESIDUAL) { HR_DISPATCH(HR_EPI_RESIDUAL) }
  else { HR_DISPATCH(HR_EPI_SWIGLU) }
#undef HR_DISPATCH
}

// Head: zsplit bf16 [2n, D] (hi rows then lo rows), W bf16 [N, D] -> fp32 [n, N]
void launch_head_gemm(const void* zsplit, int n, const void* w, int N, int D, float* out,
                      hipStream_t st) {
  EpiArgs e{};
  e.epi = HR_EPI_HEAD;
  e.out = out;
  e.ldo = N;
  e.hilo_rows = n;
  const int M = 2 * n;
  const int blocks = (N + 15) / 16;
  skinny<HR_EPI_HEAD, false>(static_cast<const uint8_t*>(zsplit), static_cast<const uint8_t*>(w),
                             M, N, 2 * D, e, blocks, 1, st);
}

}  // namespace hr
