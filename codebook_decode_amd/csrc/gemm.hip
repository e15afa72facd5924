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
//  * skinny (M <= 16; the head GEMM up to 64 rows): weight streaming.  Above 16
//    rows the tiled kernel wins (M = 64, the layer's four projections: 93 us
//    tiled against 129 us skinny, whose activation traffic per workgroup is
//    M / 16 times its weight traffic).  A workgroup owns 16 output columns
//    (16 gate + 16 up for SwiGLU; 32 for the bf16 and residual epilogues at
//    M <= 16, so each activation fragment serves twice the weight rows) and
//    its wavefronts split K; every lane streams
//    32 contiguous bytes of a weight row per step (16 rows x 128 B per wave, so
//    whole cache lines), the activation rows come from L2.  Cross-workgroup
//    split-K (grid.y) is allowed for the residual epilogue, reduced with fp32
//    atomics into h.  Wave partials are reduced in LDS in a fixed order.
//    MFMA v_mfma_f32_16x16x32_bf16 / _fp8_fp8 with M padded to 16: lane l holds
//    row/col l%16 and 8 consecutive k of lane group l/16; since A and B use the
//    same k placement, any consistent assignment of memory k to (lane group,
//    slot) is a valid contraction, which lets each lane read contiguous bytes.
//  * tiled (M > 64): BM x BN output tile per workgroup of WM x WN wavefronts,
//    32x32 MFMA blocks, K in slabs of 64 or 128 bytes per row copied HBM -> LDS
//    by global_load_lds (no register round trip) through a multi-stage ring,
//    XOR-swizzled so fragment reads are free of bank conflicts, one barrier per
//    slab, fragment reads of the next slab interleaved with this slab's MFMAs.
#include <algorithm>
#include "common.h"
#include "launch.h"
#include "rope_math.h"


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
// 16 bytes of A times 16 bytes of B along k: one fp16 MFMA (B already in
// fp16), one bf16 MFMA, or two fp8 MFMAs.
template <bool FP8, bool F16>
__device__ __forceinline__ floatx4 mma16(u32x4 a, u32x4 b, floatx4 c) {
  if constexpr (FP8) {
    c = mfma_fp8(a[0], a[1], b[0], b[1], c);
    return mfma_fp8(a[2], a[3], b[2], b[3], c);
  } else if constexpr (F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  } else {
    return mfma_bf16(a, b, c);
  }
}

// 32 x 32 output block over one K slab: NC 16-byte chunks of its row of A and
// of B per lane.  fp16 (A fp16, B converted from bf16 before the call): chunk c
// feeds one v_mfma_f32_32x32x16_f16; e4m3:
// chunks (2m, 2m+1) feed one v_mfma_scale_f32_32x32x64_f8f6f4 (format 0 = e4m3
// on both sides, unit scale) on those 32 contiguous bytes.  The 32x32 forms
// issue at twice the rate of the 16x16 ones on gfx950 (measured 2.16 vs 1.24
// PFLOP/s bf16).
template <bool FP8, int NC>
__device__ __forceinline__ floatx16 mma32(const u32x4 (&a)[NC], const u32x4 (&b)[NC], floatx16 c) {
  if constexpr (FP8) {
    typedef int intx8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int m = 0; m < NC / 2; ++m) {
      intx8 av, bv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = int(a[2 * m][i]); av[4 + i] = int(a[2 * m + 1][i]);
        bv[i] = int(b[2 * m][i]); bv[4 + i] = int(b[2 * m + 1][i]);
      }
      c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
    }
    return c;
  } else {
#pragma unroll
    for (int m = 0; m < NC; ++m)
      c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[m]), __builtin_bit_cast(f16x8, b[m]),
                                                 c, 0, 0, 0);
    return c;
  }
}

// MXFP4 32 x 32 block over one 128-value K slab: chunk m (16 B = 32 E2M1
// values of k-half h of MFMA m) feeds v_mfma_scale_f32_32x32x64_f8f6f4 with
// format 4 (E2M1) on both sides; the lane's scale dword holds the E8M0 bytes
// of blocks 0..3 of the slab for its row, and MFMA m takes block 2m + h (lane
// layout and scale semantics checked on the device against a CPU model)
__device__ __forceinline__ floatx16 mma32_mx(const u32x4 (&a)[2], const u32x4 (&b)[2], uint32_t sa, uint32_t sb,
                                             int h, floatx16 c) {
  typedef int intx8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    // E2M1 operands use the low 4 dwords of the 8-dword tuple; the high half is
    // not read, so it holds the other chunk (no zero registers, fewer moves)
    const int o = 1 - m;
    intx8 av = {int(a[m][0]), int(a[m][1]), int(a[m][2]), int(a[m][3]),
                int(a[o][0]), int(a[o][1]), int(a[o][2]), int(a[o][3])};
    intx8 bv = {int(b[m][0]), int(b[m][1]), int(b[m][2]), int(b[m][3]),
                int(b[o][0]), int(b[o][1]), int(b[o][2]), int(b[o][3])};
    const int sh = 8 * (2 * m + h);
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, int((sa >> sh) & 0xFFu), 0,
                                                        int((sb >> sh) & 0xFFu));
  }
  return c;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// value of lane (lane ^ 1) / (lane ^ 2) / the 8-lane mirror / the 16-lane
// mirror, by DPP (no LDS-pipe shuffle)
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false); }
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) { return __int_as_float(dpp_i<CTRL>(__float_as_int(v))); }
// max over the 32 lanes of a half-wave: quad swaps, 8- and 16-lane mirrors, then lane ^ 16
__device__ __forceinline__ float half_wave_max(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v));     // quad_perm(1, 0, 3, 2)
  v = fmaxf(v, dpp_f<0x4e>(v));     // quad_perm(2, 3, 0, 1)
  v = fmaxf(v, dpp_f<0x141>(v));    // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));    // row_mirror
  return fmaxf(v, __shfl_xor(v, 16, kWave));
}

struct EpiArgs {
  int epi;            // hr_epilogue
  void* out;          // fp32 [M,N] | fp32 [M,N] (+=) | act [M,F] | fp32 logits
  int ldo;            // leading dimension of out (elements)
  float x_scale;      // FP8: activation scale
  const float* w_scale;  // FP8: per-output-channel weight scale (N)
  float out_inv;      // SwiGLU FP8 output: 1 / activation scale of the next GEMM
  int out_fp8;        // SwiGLU output in e4m3
  int F;              // SwiGLU width (gate rows [0,F), up rows [F,2F))
  int hilo_rows;      // head: rows [0,h) hold hi, [h,2h) lo terms; out = hi + lo
  // RESIDUAL with split-K (ksplit > 1): split kz writes its fp32 partial to
  // part + kz * part_stride (row-major, ld = ldo) with plain stores; the caller
  // sums the splits in a fixed order (residual_norm_kernel).  ksplit == 1 adds
  // into out in place (one writer per element).  No atomics: the result does
  // not depend on the order in which workgroups finish.
  float* part;
  size_t part_stride;
  // F32 / RESIDUAL / fp16 SwiGLU outputs may be stored as 16-byte row chunks
  // (out and part 16-byte aligned, the output width and ldo whole chunks:
  // always so through the entry points, which require aligned buffers and N
  // a multiple of 16; the element-wise stores remain for the e4m3 SwiGLU
  // output and the MXFP4 residual tiles)
  int vec_store;
  // MXFP4 operands: block scales in the slab-interleaved layout [K/128][ld][4]
  QkvRope qr;            // HR_EPI_QKV_ROPE: where step A3 writes, its weights and tables
  const uint8_t* mx_sa;  // A scales, ld = mx_lda (M rounded up to the 256-row tile)
  const uint8_t* mx_sb;  // B scales, ld = N
  int mx_lda;
  uint8_t* mx_out_s;     // SwiGLU MXFP4 output: scales of the [M, F] product, ld = mx_ldo
  int mx_ldo;
};

// value of one product element after the dtype scale
template <bool FP8>
__device__ __forceinline__ float scaled(const EpiArgs& e, float acc, int n) {
  if constexpr (FP8) return acc * e.x_scale * e.w_scale[n];
  return acc;
}

// ============================================================== skinny kernel
// CB: 16-column blocks per workgroup (non-SwiGLU epilogues); SwiGLU always
// takes the gate block and the matching up block
// PK: fp16 weights in the slab-major layout of pack_weight_kernel (a lane's
// 32 bytes of a 128-byte step lie in 64-byte slab 2 step + g / 2 of its row).
template <int WAVES, int MB, int EPI, bool FP8, int U, int CB, bool PK = false>
__global__ __launch_bounds__(WAVES * 64) void gemm_skinny_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, int M, int N, int K_bytes,
    EpiArgs e) {
  constexpr int NB = (EPI == HR_EPI_SWIGLU) ? 2 : CB;  // weight row blocks per workgroup
  static_assert(EPI != HR_EPI_HEAD || CB == 1, "head epilogue: one column block");
  static_assert(!PK || (!FP8 && EPI != HR_EPI_HEAD), "packed weights: fp16 projections");
  // fp16 activations times bf16 weights converted to fp16; the head's split
  // bf16 rows (hi + lo) meet the bf16 weights directly
  constexpr bool kF16 = !FP8 && EPI != HR_EPI_HEAD;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cb = blockIdx.x;
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
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      wrow[nb] = (cb * NB + nb) * 16 + rc;
      wok[nb] = wrow[nb] < N;
    }
  }
  // packed rows: the gate/up rows interleave in 32-row blocks (gate rows
  // 32p.., then up rows 32p..); other matrices keep their row order
  int prow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (EPI == HR_EPI_SWIGLU) {
      const int a = cb * 16 + rc;
      prow[nb] = (a >> 5) * 64 + (nb ? 32 : 0) + (a & 31);
    } else {
      prow[nb] = wrow[nb];
    }
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
  // U steps of 128 bytes per wave in flight; the last batch is predicated, so
  // a wave whose share is at most U steps issues all its loads at once
  for (int s = s_lo + wave; s < s_hi; s += U * WAVES) {
    u32x4 bw[U][NB][2], ax[U][MB][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = s + u * WAVES;
      const bool sok = st < s_hi;
      const size_t kb = size_t(sok ? st : s) * 128 + g * 32;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4* p;
        if constexpr (PK)
          p = reinterpret_cast<const u32x4*>(
              w + (size_t(2 * (sok ? st : s) + (g >> 1)) * size_t(N) + size_t(prow[nb])) * 64 + (g & 1) * 32);
        else
          p = reinterpret_cast<const u32x4*>(w + size_t(wrow[nb]) * K_bytes + kb);
        bw[u][nb][0] = (wok[nb] && sok) ? p[0] : zero;
        bw[u][nb][1] = (wok[nb] && sok) ? p[1] : zero;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = mb * 16 + rc;
        const u32x4* p = reinterpret_cast<const u32x4*>(x + size_t(row) * K_bytes + kb);
        ax[u][mb][0] = (row < M && sok) ? p[0] : zero;
        ax[u][mb][1] = (row < M && sok) ? p[1] : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 b0 = (kF16 && !PK) ? bf8_to_f16x8(bw[u][nb][0]) : bw[u][nb][0];
        const u32x4 b1 = (kF16 && !PK) ? bf8_to_f16x8(bw[u][nb][1]) : bw[u][nb][1];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[nb][mb] = mma16<FP8, kF16>(ax[u][mb][0], b0, acc[nb][mb]);
          acc[nb][mb] = mma16<FP8, kF16>(ax[u][mb][1], b1, acc[nb][mb]);
        }
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
    if constexpr (EPI == HR_EPI_SWIGLU) {
      const int col = cb * 16 + (ln & 15);
      if (row < M) {
        const float gt = scaled<FP8>(e, v[0], col);
        const float up = scaled<FP8>(e, v[NB - 1], e.F + col);
        const float a = silu(gt) * up;
        if (e.out_fp8)
          static_cast<uint8_t*>(e.out)[size_t(row) * e.ldo + col] = uint8_t(f2e4m3(a * e.out_inv));
        else
          static_cast<uint16_t*>(e.out)[size_t(row) * e.ldo + col] = uint16_t(f2h(a));
      }
    } else {
#pragma unroll
     for (int nb = 0; nb < NB; ++nb) {
      const int col = (cb * NB + nb) * 16 + (ln & 15);
      if (col >= N) continue;
      if constexpr (EPI == HR_EPI_F32) {
        if (row < M) static_cast<float*>(e.out)[size_t(row) * e.ldo + col] = scaled<FP8>(e, v[nb], col);
      } else if constexpr (EPI == HR_EPI_RESIDUAL) {
        if (row < M) {
          float* o = static_cast<float*>(e.out) + size_t(row) * e.ldo + col;
          if (ksplit == 1) *o += scaled<FP8>(e, v[nb], col);
          else e.part[size_t(kz) * e.part_stride + size_t(row) * e.ldo + col] = scaled<FP8>(e, v[nb], col);
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
}

// ============================================================== tiled kernel
// BM x BN output tile per workgroup of WM x WN wavefronts; each wavefront owns a
// (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks.  K advances in 64-byte slabs
// (32 bf16 or 64 e4m3 values; 128-byte slabs for some small-M shapes) copied
// global -> LDS directly (global_load_lds_dwordx4: lane i of a wave writes 16 B
// at LDS base + 16 i) through a ring of STAGES slabs.  A slab holds BM rows of
// A and BN rows of B; the 16-byte chunks of a row are XOR-swizzled (swz below)
// so that every 16-lane phase of a fragment read hits 16 distinct bank groups
// (SQ_LDS_BANK_CONFLICT reads 0).  The swizzle is applied on the global side:
// each lane fetches the chunk its LDS slot must hold.  One barrier per slab:
// after it every wave's copies of slab s have
// landed and every wave is done with slab s-1, whose slot is refilled with slab
// s+STAGES-1.
// LDS chunk swizzle for slabs of SB bytes per row.  gfx950's LDS has 64 banks
// of 4 bytes (a 256-byte bank line) and serves a ds_read_b128 16 lanes at a
// time; the 16 lanes of one phase read one logical chunk of 16 consecutive
// rows, so those must fall in 16 distinct 16-byte bank groups.  64-byte rows
// (4 to a bank line) put chunk c of row r at c ^ ((r >> 2) & 3); 128-byte rows
// (2 to a bank line) at c ^ ((r >> 1) & 7).
template <int SB>
__device__ __forceinline__ int swz(int row) {
  if constexpr (SB == 64) return (row >> 2) & 3;
  else return (row >> 1) & 7;
}

__device__ __forceinline__ void lds_copy16(const uint8_t* g, uint8_t* lds_base) {
  // generic -> local address-space cast (not an integer truncation)
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(g),
                                   (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

// wait until at most N of this thread's vector-memory loads are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait for every outstanding LDS access of this wave (lgkmcnt 0), nothing else
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// Workgroup barrier without a memory fence: __syncthreads() would also wait for
// every outstanding global load (vmcnt(0)) and drain the slab pipeline.  The
// LDS-DMA copies this barrier publishes were already waited for by wait_vm;
// the empty asm keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int LPS, int P>
__device__ __forceinline__ void wait_pending(int pending) {
  if constexpr (P == 0) {
    wait_vm<0>();
  } else {
    if (pending >= P) wait_vm<P * LPS>();
    else wait_pending<LPS, P - 1>(pending);
  }
}
template <int LPS, int STAGES>
__device__ __forceinline__ void wait_stages(int pending) {
  // `pending` slabs issued after the one needed may stay in flight
  static_assert(STAGES >= 3 && (STAGES - 2) * LPS < 64, "vmcnt range");
  wait_pending<LPS, STAGES - 2>(pending);
}

template <int BM, int BN, int WM, int WN, int STAGES, int SB = 64>
struct TileCfg {
  static_assert(SB == 64 || SB == 128, "slab depth");
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kIM = BM / WM / 32;                  // 32-row blocks per wave
  static constexpr int kJN = BN / WN / 32;                  // 32-col blocks per wave
  static constexpr int kChunks = SB / 16;                   // 16-byte chunks per row
  static constexpr int kRowsPerCopy = 1024 / SB;            // rows per 1 KB wave copy
  static constexpr int kWaves = WM * WN;
  static constexpr int kCopies = (BM + BN) / kRowsPerCopy;  // 1 KB copies per slab
  static constexpr int kFull = kCopies / kWaves;            // whole copies per wave
  static constexpr int kRem = kCopies % kWaves;             // left over: one partial copy per wave
  static constexpr int kPartLanes = kRem * 64 / kWaves;     // lanes of each wave's partial copy
  static constexpr int kLPS = kFull + (kRem ? 1 : 0);       // copy instructions per wave per slab
  static constexpr int kSlabA = BM * SB, kSlabB = BN * SB;
  static constexpr size_t kLds = size_t(STAGES) * (kSlabA + kSlabB);
  static_assert(BM % kRowsPerCopy == 0 && BN % kRowsPerCopy == 0, "whole copies per operand");
  static_assert(kRem * 64 % kWaves == 0, "left-over copies split evenly over the waves");
  static_assert(kRem == 0 || kFull * kWaves >= BM / kRowsPerCopy, "partial copies lie in B");
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "tile shape");
};

// MX: E2M1 operands with E8M0 block scales (FP8 false).  The scales ride the
// slab ring: per slab the tile's BM + BN rows x 4 scale bytes (A rows, then B
// rows) go in kSc 1-KB copies, copy c by wave c (lane l: rows 4l .. 4l+3 of
// that KB; lanes past the last row repeat row 0 into the pad), so those waves
// issue one copy more per slab and wait for one more.
// PK: fp16 weights in the slab-major layout of pack_weight_kernel (no
// conversion; a B tile's rows of one 64-byte slab are one contiguous run).
template <int EPI, bool FP8, int BM, int BN, int WM, int WN, int STAGES, int SB, bool MX = false, bool PK = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tiled_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, int M, int N, int K_bytes,
    int tiles_m, int n_tiles, EpiArgs e) {
  static_assert(!PK || (!FP8 && !MX), "packed weights are fp16");
  using C = TileCfg<BM, BN, WM, WN, STAGES, SB>;
  constexpr int IM = C::kIM, JN = C::kJN, LPS = C::kLPS, NC = C::kChunks / 2;
  static_assert(EPI != HR_EPI_SWIGLU || JN % 2 == 0, "SwiGLU waves hold gate/up block pairs");
  constexpr int kSc = MX ? (BM + BN + 255) / 256 : 0;   // scale copies per slab
  static_assert(!MX || (!FP8 && SB == 64 && WM * WN >= kSc && C::kRem == 0), "MXFP4: 128-value (64-byte) slabs");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* sA = smem;                                   // [STAGES][BM rows][64 B]
  uint8_t* sB = smem + STAGES * C::kSlabA;              // [STAGES][BN rows][64 B]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  uint8_t* sS = smem + STAGES * (C::kSlabA + C::kSlabB);   // MX: [STAGES][kSc KB: A rows, B rows] scales
  // XCD-aware order: consecutive workgroup ids go round-robin over the 8 XCDs;
  // give each XCD a contiguous run of tiles (XCD x: n/8 of them, one more for
  // x < n % 8) so the m-tiles that share a weight tile are served by one L2
  int bid = blockIdx.x;
  {
    const int q8 = n_tiles >> 3, r8 = n_tiles & 7, xcd = bid & 7;
    bid = xcd * q8 + min(xcd, r8) + (bid >> 3);
  }
  // grouped order: runs of GM m-tiles sweep n together, so the tiles running
  // at once on one XCD share a few A and B panels in its L2
  constexpr int GM = 4;
  const int group = bid / (GM * (n_tiles / tiles_m));
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_group = bid - group * GM * (n_tiles / tiles_m);
  const int tm = first_m + in_group % gm, tn = in_group / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  // this wave's LPS copies per slab over the slab's 16-byte chunks (A rows,
  // then B rows): whole copy j takes chunks 64 (wave + j waves) + lane; when
  // the copies do not split evenly, the left-over ones (all in B) are shared
  // out as one partial copy per wave of kPartLanes lanes.  Lane i of a copy
  // fills LDS chunk (first chunk of the copy) + i of its operand.  Sources are
  // 32-bit byte offsets from x or w (the host keeps both operands under 2 GB).
  uint32_t src[LPS];
  int dst_off[LPS];
#pragma unroll
  for (int j = 0; j < LPS; ++j) {
    const bool part = C::kRem > 0 && j == C::kFull;
    const int first = part ? C::kFull * C::kWaves * 64 + wave * C::kPartLanes : (wave + j * C::kWaves) * 64;
    const int ln = part ? min(lane, C::kPartLanes - 1) : lane;
    const bool is_a = first < BM * C::kChunks;
    const int op_first = is_a ? first : first - BM * C::kChunks;   // first chunk within the operand
    const int chunk = op_first + ln;
    const int row = chunk / C::kChunks, pc = chunk % C::kChunks;
    const int lc = pc ^ swz<SB>(row);
    dst_off[j] = is_a ? op_first * 16 : STAGES * C::kSlabA + op_first * 16;
    if (is_a) {
      src[j] = uint32_t(min(m0 + row, M - 1)) * uint32_t(K_bytes) + lc * 16;
    } else {
      int br;
      if constexpr (EPI == HR_EPI_SWIGLU && !PK) {
        // 32-row blocks of the B tile alternate gate / up rows of the same
        // activation columns, so each wave holds a gate block and its up block
        // (packed weights hold their rows in that order already)
        const int blk = row >> 5, off = row & 31;
        const int a0 = min((n0 >> 1) + (blk >> 1) * 32 + off, e.F - 1);   // act column
        br = (blk & 1) ? e.F + a0 : a0;
      } else {
        br = min(n0 + row, N - 1);
      }
      if constexpr (PK)   // chunk lc of the row: 64-byte slab lc / 4 of this SB-byte slab
        src[j] = uint32_t(lc >> 2) * uint32_t(N) * 64u + uint32_t(br) * 64u + (lc & 3) * 16;
      else
        src[j] = uint32_t(br) * uint32_t(K_bytes) + lc * 16;
    }
  }
  // MX scale copy of this wave (wave < kSc): lane l carries combined rows
  // q = 256 wave + 4l .. +3 (4 bytes each): A rows below BM, then B rows
  // (mapped as the B copies), past BM + BN a repeat of A row 0
  uint32_t s_src = 0, s_ld = 0;
  bool s_is_a = true;
  if constexpr (MX) {
    const int q = 256 * wave + 4 * lane;
    if (q < BM || q >= BM + BN) {
      s_src = uint32_t(m0 + (q < BM ? q : 0)) * 4u;
      s_ld = uint32_t(e.mx_lda) * 4u;
    } else {
      const int row = q - BM;
      int br;
      if constexpr (EPI == HR_EPI_SWIGLU) {
        const int blk = row >> 5, off = row & 31;
        const int a0 = (n0 >> 1) + (blk >> 1) * 32 + off;
        br = (blk & 1) ? e.F + a0 : a0;
      } else {
        br = n0 + row;
      }
      s_src = uint32_t(br) * 4u;
      s_ld = uint32_t(N) * 4u;
      s_is_a = false;
    }
  }
  const int slabs_total = K_bytes / SB;
  const int kz = blockIdx.z, ksplit = gridDim.z;
  const int sl0 = (slabs_total * kz) / ksplit, sl1 = (slabs_total * (kz + 1)) / ksplit;
  const int n_slabs = sl1 - sl0;

  auto issue = [&](int slab, int stage) {
    const size_t ko = size_t(slab) * SB;
    // packed weights: slab-major, N rows x 64 bytes per 64-byte slab
    const size_t kob = PK ? size_t(slab) * (SB / 64) * size_t(N) * 64 : ko;
#pragma unroll
    for (int j = 0; j < LPS; ++j) {
      const bool is_a = dst_off[j] < STAGES * C::kSlabA;
      // a partial copy keeps lanes [0, kPartLanes) (lane 0 is always active, so
      // every wave issues LPS copies and the vmcnt waits below stay uniform)
      if (C::kRem > 0 && j == C::kFull && lane >= C::kPartLanes) continue;
      lds_copy16((is_a ? x : w) + src[j] + (is_a ? ko : kob),
                 smem + dst_off[j] + stage * (is_a ? C::kSlabA : C::kSlabB));
    }
    if constexpr (MX) {
      if (wave < kSc)
        lds_copy16((s_is_a ? e.mx_sa : e.mx_sb) + size_t(slab) * s_ld + s_src, sS + stage * (kSc * 1024) + wave * 1024);
    }
  };
  // wait until `pending` slabs issued after the needed one may still be in flight
  auto wait_slabs = [&](int pending) {
    if (MX && wave < kSc) wait_stages<LPS + 1, STAGES>(pending);
    else wait_stages<LPS, STAGES>(pending);
  };

  floatx16 acc[IM][JN];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < n_slabs) issue(sl0 + s, s);

  // a lane reads row (lane % 32) of each 32-row block, NC chunks of the slab:
  // bf16 chunk 2c + h feeds k-step c; e4m3 chunks 4m + 2h + {0, 1} feed MFMA m
  // (h = lane / 32)
  const int h = lane >> 5, r32 = lane & 31;
  const int a_row0 = wm * (BM / WM) + r32, b_row0 = wn * (BN / WN) + r32;
  auto chunk_of = [&](int c) { return FP8 ? 4 * (c >> 1) + 2 * h + (c & 1) : 2 * c + h; };
  typedef u32x4 Frag[NC];
  auto read_frags = [&](int stage, Frag (&fa)[IM], Frag (&fb)[JN], uint32_t (&sa)[IM], uint32_t (&sb)[JN]) {
    const uint8_t* A = sA + stage * C::kSlabA;
    const uint8_t* B = sB + stage * C::kSlabB;
    if constexpr (MX) {
      const uint8_t* S = sS + stage * (kSc * 1024);
#pragma unroll
      for (int i = 0; i < IM; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(S + (a_row0 + i * 32) * 4);
#pragma unroll
      for (int j = 0; j < JN; ++j) sb[j] = *reinterpret_cast<const uint32_t*>(S + (BM + b_row0 + j * 32) * 4);
    }
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const int r = b_row0 + j * 32;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        fb[j][c] = *reinterpret_cast<const u32x4*>(B + r * SB + ((chunk_of(c) ^ swz<SB>(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < IM; ++i) {
      const int r = a_row0 + i * 32;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        fa[i][c] = *reinterpret_cast<const u32x4*>(A + r * SB + ((chunk_of(c) ^ swz<SB>(r)) << 4));
    }
  };
  auto mma_slab = [&](const Frag (&fa)[IM], const Frag (&fb)[JN], const uint32_t (&sa)[IM],
                      const uint32_t (&sb)[JN]) {
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        if constexpr (MX) acc[i][j] = mma32_mx(fa[i], fb[j], sa[i], sb[j], h, acc[i][j]);
        else acc[i][j] = mma32<FP8, NC>(fa[i], fb[j], acc[i][j]);
      }
  };
  // Software pipeline: the fragments of slab it+1 are read from LDS while the
  // MFMAs of slab it run, so LDS latency hides behind MFMA work.  Slab it+1
  // must be resident one iteration early, hence STAGES-3 slabs stay in flight
  // during the wait.  Slot (it-1) % STAGES is refilled after the barrier of
  // iteration it: every wave's reads from it happened in iteration it-2.
  Frag fa0[IM], fb0[JN], fa1[IM], fb1[JN];
  uint32_t sa0[IM], sb0[JN], sa1[IM], sb1[JN];
  if (n_slabs > 0) {
    wait_slabs(min(STAGES - 2, n_slabs - 1));
    lds_barrier();
    read_frags(0, fa0, fb0, sa0, sb0);
  }
  int it = 0;
  constexpr int kReads = (IM + JN) * (NC + (MX ? 1 : 0)), kMfma = IM * JN * (FP8 ? NC / 2 : NC);
  auto step = [&](Frag (&fa)[IM], Frag (&fb)[JN], uint32_t (&sa)[IM], uint32_t (&sb)[JN], Frag (&fan)[IM],
                  Frag (&fbn)[JN], uint32_t (&san)[IM], uint32_t (&sbn)[JN]) {
    // this slab's fragments were read one MFMA burst ago: settle them here so
    // no wait lands between the next slab's reads and these MFMAs
    wait_lds();
    // fp16 mode: the bf16 weight fragments to fp16 once per slab (each serves
    // IM MFMAs), while this wave's next copies may still be landing
    if constexpr (!FP8 && !MX && !PK) {
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int c = 0; c < NC; ++c) fb[j][c] = bf8_to_f16x8(fb[j][c]);
    }
    wait_slabs(min(STAGES - 3, n_slabs - 2 - it));
    lds_barrier();
    // refill the slot of slab it - 1 (every wave finished reading it before
    // this barrier).  Issued here, ahead of the MFMAs: placed after them (in
    // program order) the copies ran a slab later, which measured a wash in the
    // 36-layer stack (QKV and O 0.2-0.4 us faster, the weight-streaming down
    // projection 1.5 us slower) though faster in isolation
    if (it + STAGES - 1 < n_slabs) issue(sl0 + it + STAGES - 1, (it + STAGES - 1) % STAGES);
    // the next slab's fragments (after the last slab: a stale slot, never
    // used), issued one-for-one between this slab's MFMAs: issue is in order,
    // so a burst of LDS reads stalled behind the copies into LDS would
    // otherwise leave the matrix pipe idle (10% on the gate/up GEMM at M=512)
    read_frags((it + 1) % STAGES, fan, fbn, san, sbn);
    mma_slab(fa, fb, sa, sb);
#pragma unroll
    for (int q = 0; q < (kReads < kMfma ? kReads : kMfma); ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    if constexpr (kMfma > kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
    if constexpr (kReads > kMfma) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kMfma, 0);
    ++it;
  };
  // unrolled by two so the current / next fragment sets are fixed registers
  while (it < n_slabs) {
    step(fa0, fb0, sa0, sb0, fa1, fb1, sa1, sb1);
    if (it < n_slabs) step(fa1, fb1, sa1, sb1, fa0, fb0, sa0, sb0);
  }

  // epilogue: 32x32 accumulator layout, lane holds column lane % 32 and rows
  // 8 (r / 4) + 4 (lane / 32) + r % 4 of its block, r = 0..15
  if constexpr (EPI == HR_EPI_QKV_ROPE) {
    // Step A3 on the tile's fp32 rows: the tile (after the dtype scale) goes
    // to LDS, then every (row, head) is handled as qknorm_rope_kv_kernel
    // handles it — d/16 lanes, lane c owning the RoPE pairs (8c + i,
    // d/2 + 8c + i), the head's sum of squares a butterfly over those lanes,
    // the same rounding — so q and the cache receive the same bits.
    static_assert(!MX && BN % 64 == 0, "whole heads of 64 or 128 per tile");
    constexpr int LDT = BN + 4;                      // padded fp32 row of the tile in LDS
    static_assert(size_t(BM) * LDT * 4 <= C::kLds, "the tile fits the slab ring");
    float* sT = reinterpret_cast<float*>(smem);
    wait_vm<0>();
    __syncthreads();                                 // every wave is done with the ring
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * (BM / WM) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const int cl = wn * (BN / WN) + j * 32 + r32;
          sT[rl * LDT + cl] = scaled<FP8>(e, acc[i][j][r], n0 + cl);
        }
    __syncthreads();
    const QkvRope& q = e.qr;
    const int d = q.d, half = d >> 1, L = d >> 4;
    const int heads = BN / d, items = BM * heads * L;
    const int c = tid % L;
    const uint16_t* qw = static_cast<const uint16_t*>(q.qw);
    const uint16_t* kw = static_cast<const uint16_t*>(q.kw);
    const u32x4 wq0 = *reinterpret_cast<const u32x4*>(qw + 8 * c);
    const u32x4 wq1 = *reinterpret_cast<const u32x4*>(qw + half + 8 * c);
    const u32x4 wk0 = *reinterpret_cast<const u32x4*>(kw + 8 * c);
    const u32x4 wk1 = *reinterpret_cast<const u32x4*>(kw + half + 8 * c);
    // rounds of C::kThreads items, every lane in every round (the butterfly)
    for (int base = 0; base < items; base += C::kThreads) {
      const int it = base + tid;
      const bool ok = it < items;
      const int rh = ok ? it / L : 0;
      const int rl = rh / heads, hi = rh % heads;
      const float* row = sT + rl * LDT + hi * d;
      const F8 lo = F8{*reinterpret_cast<const floatx4*>(row + 8 * c), *reinterpret_cast<const floatx4*>(row + 8 * c + 4)};
      const F8 up = F8{*reinterpret_cast<const floatx4*>(row + half + 8 * c),
                       *reinterpret_cast<const floatx4*>(row + half + 8 * c + 4)};
      const float ss = group_sum(pairs_sumsq(lo, up), L);
      const int t = m0 + rl;
      if (!ok || t >= M) continue;
      const int hidx = (n0 + hi * d) / d;            // head among q, k, v heads
      const int sq = find_seq(q.cu, q.n_seq, t);
      const int ti = t - q.cu[sq];
      const bool wkv = q.causal || ti < q.used_keys[sq];
      const long long crow = (long long)q.cache_slot[sq] * q.capacity + q.start_pos[sq] + ti;
      if (hidx < q.Hq + q.Hkv) {
        const bool is_q = hidx < q.Hq;
        if (!is_q && !wkv && !q.k16) continue;
        const float inv = 1.0f / __builtin_sqrtf(ss / float(d) + q.eps);
        const float* cs = q.rope + size_t(t) * d + 8 * c;
        F8 o0, o1;
        rope_pairs(lo, up, is_q ? wq0 : wk0, is_q ? wq1 : wk1, inv, cs, cs + half, o0, o1);
        if (is_q) {
          uint16_t* dst = static_cast<uint16_t*>(q.q_out) + (size_t(t) * q.Hq + hidx) * d;
          *reinterpret_cast<u32x4*>(dst + 8 * c) = pack8_f16(o0);
          *reinterpret_cast<u32x4*>(dst + half + 8 * c) = pack8_f16(o1);
        } else {
          const u32x4 b0 = pack8_bf16(o0), b1 = pack8_bf16(o1);
          if (wkv) {
            uint16_t* dst = static_cast<uint16_t*>(q.kc) + (size_t(crow) * q.Hkv + (hidx - q.Hq)) * d;
            *reinterpret_cast<u32x4*>(dst + 8 * c) = b0;
            *reinterpret_cast<u32x4*>(dst + half + 8 * c) = b1;
          }
          if (q.k16) {   // the fp16 copy: the cache's bf16 values widened (exact)
            uint16_t* dst = static_cast<uint16_t*>(q.k16) + (size_t(t) * q.Hkv + (hidx - q.Hq)) * d;
            *reinterpret_cast<u32x4*>(dst + 8 * c) = bf8_to_f16x8(b0);
            *reinterpret_cast<u32x4*>(dst + half + 8 * c) = bf8_to_f16x8(b1);
          }
        }
      } else {
        const u32x4 b0 = pack8_bf16(lo), b1 = pack8_bf16(up);
        if (wkv) {
          uint16_t* dst = static_cast<uint16_t*>(q.vc) + (size_t(crow) * q.Hkv + (hidx - q.Hq - q.Hkv)) * d;
          *reinterpret_cast<u32x4*>(dst + 8 * c) = b0;
          *reinterpret_cast<u32x4*>(dst + half + 8 * c) = b1;
        }
        if (q.k16) {   // the fp16 copy: the cache's bf16 values widened (exact)
          uint16_t* dst = static_cast<uint16_t*>(q.v16) + (size_t(t) * q.Hkv + (hidx - q.Hq - q.Hkv)) * d;
          *reinterpret_cast<u32x4*>(dst + 8 * c) = bf8_to_f16x8(b0);
          *reinterpret_cast<u32x4*>(dst + half + 8 * c) = bf8_to_f16x8(b1);
        }
      }
    }
    if (q.k16) {
      // rows T..Tp-1 of the fp16 copies: zero
      for (int hi = 0; hi < heads; ++hi) {
        const int hidx = (n0 + hi * d) / d;
        if (hidx < q.Hq) continue;
        const bool is_v = hidx >= q.Hq + q.Hkv;
        uint16_t* cp = static_cast<uint16_t*>(is_v ? q.v16 : q.k16);
        const int g = hidx - q.Hq - (is_v ? q.Hkv : 0);
        for (int it = tid; it < BM * (d / 8); it += C::kThreads) {
          const int t = m0 + it / (d / 8), c8 = it % (d / 8);
          if (t < M || t >= q.Tp) continue;
          *reinterpret_cast<u32x4*>(cp + (size_t(t) * q.Hkv + g) * d + 8 * c8) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    return;
  }
  if constexpr (MX && EPI == HR_EPI_SWIGLU) {
    // silu(g) * u of one row's 32 columns of a gate/up block pair is one MX
    // block of the down projection's input: its amax over the 32 lanes of the
    // half-wave, the shared exponent, E2M1 codes, two per byte (lane pairs)
    uint8_t* oc = static_cast<uint8_t*>(e.out);
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / WM) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int jj = 0; jj < JN / 2; ++jj) {
          const int cb = (n0 >> 1) + (wn * (JN / 2) + jj) * 32;     // first column of the block
          const float a = silu(acc[i][2 * jj][r]) * acc[i][2 * jj + 1][r];
          const int ex = mx_block_exp(half_wave_max(fabsf(a)));
          const uint32_t code = e2m1_code(ldexpf(a, -ex));
          const uint32_t hi = uint32_t(dpp_i<0xb1>(int(code)));
          if (row < M && cb < e.F) {
            if ((r32 & 1) == 0) oc[size_t(row) * (e.F / 2) + ((cb + r32) >> 1)] = uint8_t(code | (hi << 4));
            if (r32 == 0) e.mx_out_s[mx_scale_off(row, cb >> 5, e.mx_ldo)] = uint8_t(ex + 127);
          }
        }
      }
    return;
  }
  // Row-chunk stores through LDS: a lane's accumulators hold one column of
  // 16 rows, so direct stores write 4 (fp32) or 2 (fp16) bytes per lane and
  // instruction.  Instead each pass of 32 rows per wave row (IM passes) goes to
  // LDS as the tile's output rows, then every thread stores 16-byte chunks of
  // them (a wave instruction covers whole rows): a quarter to an eighth of
  // the store instructions.  Same values, same bits as the direct stores.
  if constexpr (!MX && (EPI == HR_EPI_F32 || EPI == HR_EPI_RESIDUAL || EPI == HR_EPI_SWIGLU)) {
    if (e.vec_store) {
      constexpr bool SG = EPI == HR_EPI_SWIGLU;
      constexpr int EB = SG ? 2 : 4;                   // output bytes per element
      constexpr int CO = SG ? BN / 2 : BN;             // output columns of the tile
      constexpr int PR = 32 * WM;                      // tile rows per pass
      constexpr int LDR = CO * EB + 32;                // padded LDS row (bytes): the two half-waves
                                                       // (rows 4 apart) land on distinct banks
      constexpr int CPR = CO * EB / 16;                // 16-byte chunks per row
      static_assert(size_t(PR) * LDR <= C::kLds, "a pass fits the slab ring");
      static_assert((CO * EB) % 64 == 0, "whole 64-byte row segments");
      const int col0 = SG ? (n0 >> 1) : n0;            // first output column of the tile
      const int ncol = SG ? e.F : N;
      uint8_t* sE = smem;
      wait_vm<0>();                                     // no copy into the ring in flight
#pragma unroll
      for (int i = 0; i < IM; ++i) {
        __syncthreads();                                // the ring (or the previous pass) is free
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = wm * 32 + 8 * (r >> 2) + 4 * h + (r & 3);   // row within the pass
          if constexpr (SG) {
#pragma unroll
            for (int jj = 0; jj < JN / 2; ++jj) {
              const int cl = (wn * (JN / 2) + jj) * 32 + r32;
              const int col = col0 + cl;
              const int cg = min(col, e.F - 1);
              const float gt = scaled<FP8>(e, acc[i][2 * jj][r], cg);
              const float up = scaled<FP8>(e, acc[i][2 * jj + 1][r], e.F + cg);
              *reinterpret_cast<uint16_t*>(sE + lr * LDR + cl * 2) = uint16_t(f2h(silu(gt) * up));
            }
          } else {
#pragma unroll
            for (int j = 0; j < JN; ++j) {
              const int cl = wn * (BN / WN) + j * 32 + r32;
              *reinterpret_cast<float*>(sE + lr * LDR + cl * 4) = scaled<FP8>(e, acc[i][j][r], min(n0 + cl, N - 1));
            }
          }
        }
        __syncthreads();
        for (int c = tid; c < PR * CPR; c += C::kThreads) {
          const int lr = c / CPR, ch = c % CPR;
          const int row = m0 + (lr >> 5) * (BM / WM) + i * 32 + (lr & 31);
          const int col = col0 + ch * (16 / EB);
          if (row >= M || col >= ncol) continue;
          const u32x4 v = *reinterpret_cast<const u32x4*>(sE + lr * LDR + ch * 16);
          if constexpr (SG) {
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(e.out) + size_t(row) * e.ldo + col) = v;
          } else if constexpr (EPI == HR_EPI_F32) {
            *reinterpret_cast<u32x4*>(static_cast<float*>(e.out) + size_t(row) * e.ldo + col) = v;
          } else if (ksplit == 1) {
            floatx4* o = reinterpret_cast<floatx4*>(static_cast<float*>(e.out) + size_t(row) * e.ldo + col);
            const floatx4 a = __builtin_bit_cast(floatx4, v);
            const floatx4 b = *o;
            *o = floatx4{b[0] + a[0], b[1] + a[1], b[2] + a[2], b[3] + a[3]};
          } else {
            *reinterpret_cast<u32x4*>(e.part + size_t(kz) * e.part_stride + size_t(row) * e.ldo + col) = v;
          }
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < IM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * (BM / WM) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row >= M) continue;
      if constexpr (EPI == HR_EPI_SWIGLU) {
#pragma unroll
        for (int jj = 0; jj < JN / 2; ++jj) {
          const int col = (n0 >> 1) + (wn * (JN / 2) + jj) * 32 + r32;
          if (col < e.F) {
            const float gt = scaled<FP8>(e, acc[i][2 * jj][r], col);
            const float up = scaled<FP8>(e, acc[i][2 * jj + 1][r], e.F + col);
            const float a = silu(gt) * up;
            if (e.out_fp8)
              static_cast<uint8_t*>(e.out)[size_t(row) * e.ldo + col] = uint8_t(f2e4m3(a * e.out_inv));
            else
              static_cast<uint16_t*>(e.out)[size_t(row) * e.ldo + col] = uint16_t(f2h(a));
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          const int col = n0 + wn * (BN / WN) + j * 32 + r32;
          if (col >= N) continue;
          const float v = scaled<FP8>(e, acc[i][j][r], col);
          if constexpr (EPI == HR_EPI_F32) {
            static_cast<float*>(e.out)[size_t(row) * e.ldo + col] = v;
          } else {
            if (ksplit == 1) static_cast<float*>(e.out)[size_t(row) * e.ldo + col] += v;
            else e.part[size_t(kz) * e.part_stride + size_t(row) * e.ldo + col] = v;
          }
        }
      }
    }
  }
}

// ============================================================== dispatch
// 16-column blocks per workgroup for the bf16 / residual epilogues at M <= 16:
// two blocks read each activation fragment for twice the weight rows
constexpr int kSkinnyCB = 2;

template <int EPI>
constexpr int skinny_cb(int mb) { return (mb == 1 && (EPI == HR_EPI_F32 || EPI == HR_EPI_RESIDUAL)) ? kSkinnyCB : 1; }

template <int EPI, bool FP8, bool PK = false>
static void skinny(const uint8_t* x, const uint8_t* w, int M, int N, int Kb, const EpiArgs& e,
                   int blocks, int ksplit, hipStream_t st) {
  dim3 grid(blocks, ksplit);
  const int mb = (M + 15) / 16;
  // 128-byte steps per wave (8 waves, the largest split)
  const int steps = Kb / 128;
  const int spw = ((steps + ksplit - 1) / ksplit + 7) / 8;
  constexpr int CB1 = (EPI == HR_EPI_F32 || EPI == HR_EPI_RESIDUAL) ? kSkinnyCB : 1;
  constexpr int NB1 = (EPI == HR_EPI_SWIGLU) ? 2 : CB1;
  if (mb == 1) {
    // all of a wave's steps in one batch when they fit (5 steps x NB = 1 block
    // measured faster than 4 + 1; at NB = 2 the 5-step batch costs occupancy,
    // except for the fp32 epilogue, whose grid (the merged QKV rows: 192
    // workgroups) has one workgroup per CU anyway: M = 13, 9.4 -> 8.9 us)
    if (spw <= 2) gemm_skinny_kernel<8, 1, EPI, FP8, 2, CB1, PK><<<grid, 512, 0, st>>>(x, w, M, N, Kb, e);
    else if (spw == 3) gemm_skinny_kernel<8, 1, EPI, FP8, 3, CB1, PK><<<grid, 512, 0, st>>>(x, w, M, N, Kb, e);
    else if (spw == 5 && (NB1 == 1 || EPI == HR_EPI_F32))
      gemm_skinny_kernel<8, 1, EPI, FP8, 5, CB1, PK><<<grid, 512, 0, st>>>(x, w, M, N, Kb, e);
    else gemm_skinny_kernel<8, 1, EPI, FP8, 4, CB1, PK><<<grid, 512, 0, st>>>(x, w, M, N, Kb, e);
  } else if (EPI == HR_EPI_SWIGLU) {
    if (mb == 2) gemm_skinny_kernel<4, 2, EPI, FP8, 4, 1, PK><<<grid, 256, 0, st>>>(x, w, M, N, Kb, e);
    else gemm_skinny_kernel<4, 4, EPI, FP8, 4, 1, PK><<<grid, 256, 0, st>>>(x, w, M, N, Kb, e);
  } else {
    if (mb == 2) gemm_skinny_kernel<8, 2, EPI, FP8, 4, 1, PK><<<grid, 512, 0, st>>>(x, w, M, N, Kb, e);
    else gemm_skinny_kernel<4, 4, EPI, FP8, 4, 1, PK><<<grid, 256, 0, st>>>(x, w, M, N, Kb, e);
  }
}

template <int EPI, bool FP8, int BM, int BN, int WM, int WN, int STAGES, int SB, bool MX = false, bool PK = false>
static void tiled_cfg(const uint8_t* x, const uint8_t* w, int M, int N, int Kb, const EpiArgs& e,
                      int ksplit, hipStream_t st) {
  using C = TileCfg<BM, BN, WM, WN, STAGES, SB>;
  constexpr size_t kLds = C::kLds + (MX ? size_t(STAGES) * 1024 * ((BM + BN + 255) / 256) : 0);
  const int tiles_m = (M + BM - 1) / BM;
  const int ncols = (EPI == HR_EPI_SWIGLU) ? 2 * e.F : N;
  const int tiles_n = (ncols + BN - 1) / BN;
  const int n_tiles = tiles_m * tiles_n;
  auto kern = gemm_tiled_kernel<EPI, FP8, BM, BN, WM, WN, STAGES, SB, MX, PK>;
  if (kLds > 65536) {
    // above the 64 KB default dynamic-LDS limit: raised once per kernel (a
    // thread-safe static); a refusal surfaces as the launch's error
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(kLds));
    (void)raised;
  }
  dim3 grid(n_tiles, 1, ksplit);
  kern<<<grid, C::kThreads, kLds, st>>>(x, w, M, N, Kb, tiles_m, n_tiles, e);
}

// Split-K factor that fills the 256 CUs for the residual projections (the
// splits' partials are summed by the caller), or the given one; launched only
// when `go` (otherwise this only plans the factor).
template <int EPI, bool FP8, int BM, int BN, int WM, int WN, int STAGES, int SB = 64, bool MX = false, bool PK = false>
static int tiled_fill(const uint8_t* x, const uint8_t* w, int M, int N, int Kb, const EpiArgs& e,
                      hipStream_t st, bool go, int ks_force = 0) {
  const int ncols = (EPI == HR_EPI_SWIGLU) ? 2 * e.F : N;
  const int tiles = ((M + BM - 1) / BM) * ((ncols + BN - 1) / BN);
  int ks = 1;
  if (EPI == HR_EPI_RESIDUAL && tiles < 256) ks = (256 + tiles - 1) / tiles;
  if (EPI == HR_EPI_RESIDUAL && ks_force > 0) ks = ks_force;
  const int max_ks = Kb / SB / 4 > 0 ? Kb / SB / 4 : 1;   // >= 4 slabs per split
  if (ks > max_ks) ks = max_ks;
  if (go) tiled_cfg<EPI, FP8, BM, BN, WM, WN, STAGES, SB, MX, PK>(x, w, M, N, Kb, e, ks, st);
  return ks;
}

// Tile configuration of the large-M GEMM, per projection and M range, from
// sweeps of 12-13 tile shapes, slab depths and split-K factors on MI355X with
// the 4B layer's shapes (M = 128, 256, 512, 4192 bf16; M = 544 e4m3; M = 32
// and 64, the batched decode step, from a sweep of 4).  Small M
// wants small tiles (more workgroups than CUs: QKV at M = 128 runs 39 -> 20 us
// going from 128x128 to 64x64 tiles with 128-byte slabs); large M wants the
// 256x256 tile (LDS traffic per MFMA).  Split-K fills the grid for the
// residual projections.  Re-swept at M = 512 once the LDS swizzle and the
// interleaved fragment reads were in: bf16 QKV and O on 128x128 tiles of 8
// waves with 128-byte slabs (QKV 32.6 us against 48.8 on 64x128, O 27.5
// against 34.1 on 128x64; gate/up and down keep their tiles, every alternative
// tried was slower); e4m3 at M = 544: QKV and gate/up on the same 128x128
// tiles (22.5 against 30.7 us on 64x128, 58.1 against 60.3 on 256x256), O and
// down on 64x64 with 128-byte slabs (26.1 / 44.6 against 28.8 / 46.0 on
// 128x64); at M = 4096 the residual projections on the
// same 128x128 tiles (O 140 us against 156 on 256x256, down 284 against 289,
// QKV stays on 256x256: 153 against 177); at M = 128 gate/up on 8 waves (35.9
// against 38.0 us), down 128x64 and O 64x64 with 128-byte slabs (32.5 / 14.1
// against 34.7 / 17.0).
// bf16 weights reach the fp16 MFMAs converted in registers, once per B
// fragment and slab, so the 8-wave tiles stand their waves 2 x 4 (each wave
// 2x the A rows and half the B columns of a 4 x 2 layout: half the
// conversions for the same LDS reads): at 512 rows QKV 36.9 -> 31.7 us,
// O 31.4 -> 28.7, gate/up 95.4 -> 87.2, down 52.1 -> 49.0 (weights rotated
// through 4 copies).  The e4m3 tiles keep their layout (no conversion).
// Re-swept with fp16 activations at 64, 128 and 4274 rows: the down projection
// (K 9728) at up to 128 rows takes the O projection's 64 x 64 tiles with 4
// stages (2 workgroups per CU): 30.1 -> 20.8 us at 64 rows, 38.8 -> 28.3 at
// 128; every other tile stayed (256 x 128 residual tiles above 1024 rows won
// alone, O 165.7 -> 159.3 and down 330.0 -> 303.8 us at 4274 rows, but the
// 36-layer varlen batch got slower with them: 46.3 -> 49.8 ms).
template <int EPI, bool FP8, bool PK>
static int tiled(const uint8_t* x, const uint8_t* w, int M, int N, int Kb, const EpiArgs& e,
                 hipStream_t st, bool go) {
  const int K_el = FP8 ? Kb : Kb / 2;
  if constexpr (EPI == HR_EPI_SWIGLU) {
    if (M <= 64) return tiled_fill<EPI, FP8, 64, 128, 2, 2, 6, 128, false, PK>(x, w, M, N, Kb, e, st, go);
    if (M > 384) {
      if constexpr (FP8) {
        // e4m3, 385-576 rows: 192 x 256 tiles with 64-byte slabs (228
        // workgroups; the FP8 layer at 544 rows 174 -> 165 us)
        if (M <= 576) return tiled_fill<EPI, FP8, 192, 256, 2, 4, 4, 64, false, PK>(x, w, M, N, Kb, e, st, go);
        return tiled_fill<EPI, FP8, 128, 128, 4, 2, 4, 128, false, PK>(x, w, M, N, Kb, e, st, go);
      }
      // packed weights, 385-576 rows: 192-row tiles, 3 x 76 = 228 workgroups
      // for the 4B gate/up instead of 152 (M = 512: 76.9 -> 67.4 us; with the
      // in-register conversion the 192-row tile only broke even)
      if constexpr (PK) {
        if (M <= 576) return tiled_fill<EPI, FP8, 192, 256, 2, 4, 4, 64, false, PK>(x, w, M, N, Kb, e, st, go);
      }
      return tiled_fill<EPI, FP8, 256, 256, 2, 4, 4, 64, false, PK>(x, w, M, N, Kb, e, st, go);
    }
    if (M > 128) return tiled_fill<EPI, FP8, 256, 128, 4, 2, 4, 64, false, PK>(x, w, M, N, Kb, e, st, go);
    return tiled_fill<EPI, FP8, 128, 128, 4, 2, 4, 128, false, PK>(x, w, M, N, Kb, e, st, go);
  } else if constexpr (EPI == HR_EPI_F32) {
    if (M > 1024) return tiled_fill<EPI, FP8, 256, 256, 2, 4, 4, 64, false, PK>(x, w, M, N, Kb, e, st, go);
    if (M > 384) return tiled_fill<EPI, FP8, 128, 128, 2, 4, 4, 128, false, PK>(x, w, M, N, Kb, e, st, go);
    if (M > 128) return tiled_fill<EPI, FP8, 128, 64, 2, 2, 6, 128, false, PK>(x, w, M, N, Kb, e, st, go);
    if (M <= 64) return tiled_fill<EPI, FP8, 64, 32, 2, 1, 8, 128, false, PK>(x, w, M, N, Kb, e, st, go);
    return tiled_fill<EPI, FP8, 64, 64, 2, 2, 8, 128, false, PK>(x, w, M, N, Kb, e, st, go);
  } else {
    if constexpr (FP8) {
      // e4m3 O and down at 385-576 rows: 128 x 128 tiles split 2 ways (the
      // FP8 layer 165 -> 159 us against 64 x 64 unsplit)
      if (M > 384 && M <= 576) return tiled_fill<EPI, FP8, 128, 128, 2, 4, 4, 128, false, PK>(x, w, M, N, Kb, e, st, go, 2);
      if (M > 128) return tiled_fill<EPI, FP8, 64, 64, 2, 2, 4, 128, false, PK>(x, w, M, N, Kb, e, st, go);
    }
    if (M > 1024) return tiled_fill<EPI, FP8, 128, 128, 2, 4, 4, 128, false, PK>(x, w, M, N, Kb, e, st, go);
    if (M > 384) {
      // the down projection (K >= 8192) at 385-576 rows: 128 x 128 tiles split
      // 3 ways (240 workgroups at M = 512, half the partials of 256 x 128 split
      // 6 ways: GEMM + partial sum 48.7 -> 46.3 us, packed weights)
      if (K_el >= 8192 && M <= 576) return tiled_fill<EPI, FP8, 128, 128, 2, 4, 4, 128, false, PK>(x, w, M, N, Kb, e, st, go, 3);
      if (K_el >= 8192) return tiled_fill<EPI, FP8, 256, 128, 2, 4, 4, 64, false, PK>(x, w, M, N, Kb, e, st, go, 6);
      return tiled_fill<EPI, FP8, 128, 128, 2, 4, 4, 128, false, PK>(x, w, M, N, Kb, e, st, go, 3);
    }
    if (M > 128) return tiled_fill<EPI, FP8, 128, 128, 2, 2, 4, 64, false, PK>(x, w, M, N, Kb, e, st, go);
    return tiled_fill<EPI, FP8, 64, 64, 2, 2, 4, 128, false, PK>(x, w, M, N, Kb, e, st, go);
  }
}

int launch_linear(const void* x, const void* w, const float* w_scale, float x_scale, bool fp8, bool packed,
                  int M, int N, int K, int epi, void* out, float out_scale, float* part, bool go,
                  hipStream_t st) {
  EpiArgs e{};
  e.epi = epi;
  e.out = out;
  e.x_scale = x_scale;
  e.w_scale = w_scale;
  e.out_fp8 = (epi == HR_EPI_SWIGLU && fp8) ? 1 : 0;
  e.out_inv = out_scale > 0.f ? 1.0f / out_scale : 1.0f;
  e.F = N / 2;
  e.ldo = (epi == HR_EPI_SWIGLU) ? N / 2 : N;
  e.part = part;
  e.part_stride = size_t(M) * size_t(N);
  {
    const int eb = (epi == HR_EPI_SWIGLU) ? 2 : 4;
    const int width = (epi == HR_EPI_SWIGLU) ? N / 2 : N;
    const bool al = reinterpret_cast<uintptr_t>(out) % 16 == 0 && reinterpret_cast<uintptr_t>(part) % 16 == 0;
    e.vec_store = (epi == HR_EPI_F32 || epi == HR_EPI_RESIDUAL || (epi == HR_EPI_SWIGLU && !fp8)) && al &&
                  (width * eb) % 16 == 0 && (e.ldo * eb) % 16 == 0;
  }
  const int Kb = fp8 ? K : 2 * K;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  const int ncols = (epi == HR_EPI_SWIGLU) ? N / 2 : N;
  int ks = 1;
  // small batches: the residual projections split K over about 384 workgroups
  // (1.5 per CU; measured at T = 13 against 256, 512 and 768: O 8.2 us against
  // 8.7 / 8.8 / 8.7, down 14.6 against 16.7 / 15.0 / 14.9)
#define HR_DISPATCH(EPI_)                                                                     \
  if (M <= 16) {                                                                              \
    const int cbw = 16 * skinny_cb<EPI_>((M + 15) / 16);                                      \
    const int blocks = (ncols + cbw - 1) / cbw;                                               \
    if (EPI_ == HR_EPI_RESIDUAL && blocks < 256) ks = (384 + blocks - 1) / blocks;            \
    if (ks > Kb / 128) ks = Kb / 128;                                                         \
    if (go && fp8) skinny<EPI_, true>(xb, wb, M, N, Kb, e, blocks, ks, st);                   \
    else if (go && packed) skinny<EPI_, false, true>(xb, wb, M, N, Kb, e, blocks, ks, st);     \
    else if (go) skinny<EPI_, false>(xb, wb, M, N, Kb, e, blocks, ks, st);                    \
  } else {                                                                                    \
    ks = fp8 ? tiled<EPI_, true, false>(xb, wb, M, N, Kb, e, st, go)                          \
             : packed ? tiled<EPI_, false, true>(xb, wb, M, N, Kb, e, st, go)                 \
                      : tiled<EPI_, false, false>(xb, wb, M, N, Kb, e, st, go);               \
  }
  if (epi == HR_EPI_F32) { HR_DISPATCH(HR_EPI_F32) }
  else if (epi == HR_EPI_RESIDUAL) { HR_DISPATCH(HR_EPI_RESIDUAL) }
  else { HR_DISPATCH(HR_EPI_SWIGLU) }
#undef HR_DISPATCH
  return ks;
}

bool qkv_rope_fits(int M, int d) { return M > 384 && M <= 1024 && (d == 64 || d == 128); }

// 128 x 128 tiles (the F32 table's choice for these rows): a tile column
// block is one head of 128 or two of 64
bool launch_qkv_rope(const void* x, const void* w, const float* w_scale, float x_scale, bool fp8, bool packed,
                     int M, int K, const QkvRope& qr, hipStream_t st) {
  if (!qkv_rope_fits(M, qr.d)) return false;
  EpiArgs e{};
  e.epi = HR_EPI_QKV_ROPE;
  e.x_scale = x_scale;
  e.w_scale = w_scale;
  e.qr = qr;
  const int N = (qr.Hq + 2 * qr.Hkv) * qr.d;
  e.ldo = N;
  const int Kb = fp8 ? K : 2 * K;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  constexpr int E = HR_EPI_QKV_ROPE;
  if (fp8) tiled_cfg<E, true, 128, 128, 2, 4, 4, 128>(xb, wb, M, N, Kb, e, 1, st);
  else if (packed) tiled_cfg<E, false, 128, 128, 2, 4, 4, 128, false, true>(xb, wb, M, N, Kb, e, 1, st);
  else tiled_cfg<E, false, 128, 128, 2, 4, 4, 128>(xb, wb, M, N, Kb, e, 1, st);
  return true;
}

// MXFP4 x MXFP4: x codes [M, K/2] with scales (ld lda), w codes [N, K/2] with
// scales (ld N); RESIDUAL adds into fp32 out [M, N]; SWIGLU (N = 2F) writes the
// MXFP4 product: codes [M, F/2] into out, scales (ld ldo) into out_scales.
int launch_linear_mx(const uint8_t* x, const uint8_t* x_scales, int lda, const uint8_t* w,
                     const uint8_t* w_scales, int M, int N, int K, int epi, void* out, uint8_t* out_scales,
                     int ldo, float* part, bool go, hipStream_t st) {
  EpiArgs e{};
  e.epi = epi;
  e.out = out;
  e.ldo = N;
  e.F = N / 2;
  e.mx_sa = x_scales;
  e.mx_sb = w_scales;
  e.mx_lda = lda;
  e.mx_out_s = out_scales;
  e.mx_ldo = ldo;
  e.part = part;
  e.part_stride = size_t(M) * size_t(N);
  const int Kb = K / 2;
  // tiles from a sweep of the MXFP4 layer at P = 512: gate/up 128 x 128 on 8
  // waves (the layer 166 -> 156 us against 256 x 256), O and down 64 x 128
  // (-> 153 us against 128 x 64; 128 x 128 and 64 x 64 slower)
  if (epi == HR_EPI_SWIGLU)
    return tiled_fill<HR_EPI_SWIGLU, false, 128, 128, 4, 2, 4, 64, true>(x, w, M, N, Kb, e, st, go);
  if (M > 1024) return tiled_fill<HR_EPI_RESIDUAL, false, 256, 256, 4, 2, 4, 64, true>(x, w, M, N, Kb, e, st, go);
  return tiled_fill<HR_EPI_RESIDUAL, false, 64, 128, 2, 2, 4, 64, true>(x, w, M, N, Kb, e, st, go);
}

// ============================================================== weight packing
// Packed fp16 weights: W [N, K] bf16 row-major -> P [K/32][N][32] fp16: each
// 64-byte run is one row's slab of 32 K values, so the rows of a tile for one
// slab are one contiguous run.  gate_up (W = [gate; up], N = 2F): packed row
// 64 p + 32 u + r holds row u F + 32 p + r, the 32-row gate / up block order
// the SwiGLU tiles consume.  The values are converted as the bf16 path does in
// registers (bf8_to_f16x8: exact for |w| in [2^-17, 65504], round to nearest
// even below), so a packed layer computes the same products in the same order;
// a non-finite result (|w| >= 65520, inf or NaN) sets *bad.
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint16_t* __restrict__ w, int N, int K, int gate_up,
                                                          uint16_t* __restrict__ out, unsigned int* __restrict__ bad) {
  const size_t n_chunks = size_t(N) * size_t(K / 8);
  unsigned int nonfinite = 0;
  for (size_t c = size_t(blockIdx.x) * 256 + threadIdx.x; c < n_chunks; c += size_t(gridDim.x) * 256) {
    const int q = int(c & 3);                 // 8-value quarter of the 64-byte run
    const size_t run = c >> 2;
    const int pr = int(run % size_t(N)), sl = int(run / size_t(N));
    int row = pr;
    if (gate_up) {
      const int F = N / 2;
      row = ((pr >> 5) & 1) * F + 32 * (pr >> 6) + (pr & 31);
    }
    const u32x4 h = bf8_to_f16x8(*reinterpret_cast<const u32x4*>(w + size_t(row) * K + size_t(sl) * 32 + q * 8));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      nonfinite |= ((h[i] & 0x7C00u) == 0x7C00u) | (((h[i] >> 16) & 0x7C00u) == 0x7C00u);
    *reinterpret_cast<u32x4*>(out + c * 8) = h;
  }
  if (nonfinite) atomicOr(bad, 1u);
}

// the non-finite flag of pack_weight_kernel: one word per GPU (file scope, no
// allocation); packs that overlap on one GPU share it
__device__ unsigned int g_pack_bad;

int launch_pack_weight(const void* w, int N, int K, bool gate_up, void* out, hipStream_t st) {
  unsigned int* bad = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&bad), HIP_SYMBOL(g_pack_bad)) != hipSuccess) return -1;
  unsigned int h_bad = 0;
  const size_t n_chunks = size_t(N) * size_t(K / 8);
  const int blocks = int(std::min<size_t>((n_chunks + 255) / 256, 16384));
  if (hipMemcpyAsync(bad, &h_bad, sizeof(h_bad), hipMemcpyHostToDevice, st) != hipSuccess) return -1;
  pack_weight_kernel<<<blocks, 256, 0, st>>>(static_cast<const uint16_t*>(w), N, K, gate_up ? 1 : 0,
                                              static_cast<uint16_t*>(out), bad);
  if (hipGetLastError() != hipSuccess ||
      hipMemcpyAsync(&h_bad, bad, sizeof(h_bad), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return -1;
  return h_bad ? 1 : 0;
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
