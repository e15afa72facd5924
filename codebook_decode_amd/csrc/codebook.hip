// Delayed-codebook step (FlashRT pull request 141 "Stabilize Higgs Audio
// termination and prefill", Summary and Root cause): per-frame argmax of every
// codebook, delay-pattern bookkeeping (BOS fill while t < k, sticky per-codebook
// EOC, done once every codebook has emitted EOC) and the codebook-embedding sum
// that feeds the next decode step.
//
// One workgroup of 512 threads per stream.  The step is two dependent reads
// (logits, then the chosen embedding rows), so the kernel is built to have
// each read in flight at once rather than one load after another:
//  * argmax: G lanes per codebook (G = 512 / K rounded down to a power of two,
//    at most one wavefront); the row is read as aligned 16-byte units of the
//    tensor (8 bf16 or 4 fp32; a unit may straddle two rows, the elements
//    outside the row are skipped), up to kUnits units per lane issued before
//    any compare; each lane keeps (max, lowest index) over its units in
//    increasing index order and a butterfly over the G lanes picks the row's
//    first maximum;
//  * lane k applies codebook k's delay / EOC update; one lane updates the
//    frame counter and done;
//  * embedding sum: one 16-byte chunk of D per thread, the K rows loaded in
//    batches of 8 before they are added, in codebook order, in fp32, rounded
//    once to bf16.
#include "common.h"
#include "launch.h"

namespace hr {

constexpr int kCbThreads = 512;
constexpr int kUnits = 5;       // 16-byte units per lane per batch (V <= 2560 bf16 / 1280 fp32 in one batch at 64 lanes)

// value of pair unit u (elements 2u, 2u+1 of the logits tensor); the last
// unit of an odd-sized tensor holds one element
// 16-byte unit u of the logits tensor (elements [E u, E u + E), E = 8 bf16 or
// 4 fp32; the tensor is 16-byte aligned); a unit that runs past the end of the
// tensor is read element by element, the missing ones as -inf
template <bool F32>
__device__ __forceinline__ u32x4 load_unit(const void* p, size_t u, size_t total) {
  constexpr int E = F32 ? 4 : 8;
  if (size_t(E) * (u + 1) <= total) return reinterpret_cast<const u32x4*>(p)[u];
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (F32) {
      const size_t e = 4 * u + q;
      v[q] = e < total ? __float_as_uint(static_cast<const float*>(p)[e]) : 0xFF800000u;
    } else {
      const size_t e0 = 8 * u + 2 * q, e1 = e0 + 1;
      const uint32_t lo = e0 < total ? static_cast<const uint16_t*>(p)[e0] : 0xFF80u;
      const uint32_t hi = e1 < total ? static_cast<const uint16_t*>(p)[e1] : 0xFF80u;
      v[q] = lo | (hi << 16);
    }
  }
  return v;
}

template <bool F32>
__device__ __forceinline__ float unit_elem(const u32x4& v, int e) {   // e constant
  if (F32) return __uint_as_float(v[e]);
  return (e & 1) ? bf_hi(v[e >> 1]) : bf_lo(v[e >> 1]);
}

template <bool F32>
__global__ __launch_bounds__(kCbThreads) void codebook_step_kernel(
    int K, int V, int G, int bos, int eoc, const void* __restrict__ logits, size_t total,
    int32_t* __restrict__ frame, uint8_t* __restrict__ eoc_seen, uint8_t* __restrict__ done,
    int32_t* __restrict__ codes, int32_t* __restrict__ aligned, int max_frames,
    const uint16_t* __restrict__ cb_embed, int D, uint16_t* __restrict__ emb_out) {
  extern __shared__ int32_t s_code[];  // [K] argmax ids, then chosen codes; [K, 2K) seen flags
  const int b = blockIdx.x;
  const bool is_done = done[b] != 0;
  // the stream's state is read up front, with the logits, so the bookkeeping
  // below waits on no memory
  const int t = frame[b];
  for (int k = threadIdx.x; k < K; k += blockDim.x) s_code[K + k] = eoc_seen[size_t(b) * K + k];

  if (!is_done) {
    const int groups = kCbThreads / G, grp = threadIdx.x / G, gl = threadIdx.x % G;
    for (int k = grp; k < K; k += groups) {
      constexpr int E = F32 ? 4 : 8;                         // elements per unit
      const size_t base = (size_t(b) * K + k) * V;          // first element of the row
      const size_t u0 = base / E;                           // its unit
      const int off0 = int(base - u0 * E);                  // element offset within that unit
      const int nu = int((base + V + E - 1) / E - u0);      // units touching the row
      float best = -__builtin_inff();
      int bi = 0x7FFFFFFF;
      for (int ui = gl; ui < nu; ui += G * kUnits) {
        u32x4 x[kUnits];
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
          const int idx = ui + j * G;
          if (idx < nu) x[j] = load_unit<F32>(logits, u0 + idx, total);
        }
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
          const int idx = ui + j * G;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const int v = E * idx + e - off0;
            const float xv = unit_elem<F32>(x[j], e);
            if (idx < nu && v >= 0 && v < V && (xv > best || bi == 0x7FFFFFFF)) {
              best = xv;
              bi = v;
            }
          }
        }
      }
      for (int m = G >> 1; m >= 1; m >>= 1) {
        const float ob = __shfl_xor(best, m, kWave);
        const int oi = __shfl_xor(bi, m, kWave);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      if (gl == 0) s_code[k] = bi;
    }
  }
  __syncthreads();
  // delay / EOC bookkeeping: one lane per codebook, then one lane for the stream
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    int c = eoc;
    if (!is_done) {
      const size_t ks = size_t(b) * K + k;
      const bool seen = s_code[K + k] != 0;
      c = (t < k) ? bos : (seen ? eoc : s_code[k]);
      if (c == eoc && !seen) eoc_seen[ks] = 1;
      if (aligned != nullptr && t >= k && t - k < max_frames)
        aligned[(size_t(b) * max_frames + (t - k)) * K + k] = c;
      s_code[K + k] = (seen || c == eoc) ? 1 : 0;
    }
    s_code[k] = c;
    codes[size_t(b) * K + k] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0 && !is_done) {
    bool all = true;
    for (int k = 0; k < K; ++k) all = all && s_code[K + k] != 0;
    frame[b] = t + 1;
    done[b] = all ? 1 : 0;
  }

  // emb[b] = bf16( ((E[c0] + E[V+c1]) + ...) + E[(K-1)V + c_{K-1}] ), fp32 sum
  for (int d8 = threadIdx.x; d8 * 8 < D; d8 += blockDim.x) {
    float acc[8];
    for (int k0 = 0; k0 < K; k0 += 8) {
      u32x4 r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < K)
          r[j] = reinterpret_cast<const u32x4*>(cb_embed + (size_t(k0 + j) * V + s_code[k0 + j]) * D)[d8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (k0 + j >= K) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (k0 + j == 0) {
            acc[2 * q] = bf_lo(r[j][q]);
            acc[2 * q + 1] = bf_hi(r[j][q]);
          } else {
            acc[2 * q] += bf_lo(r[j][q]);
            acc[2 * q + 1] += bf_hi(r[j][q]);
          }
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf2(acc[2 * j], acc[2 * j + 1]);
    reinterpret_cast<u32x4*>(emb_out + size_t(b) * D)[d8] = o;
  }
}

void launch_codebook_step(int B, int K, int V, int bos, int eoc, bool f32, const void* logits,
                          int32_t* frame, uint8_t* eoc_seen, uint8_t* done, int32_t* codes,
                          int32_t* aligned, int max_frames, const void* cb_embed, int D,
                          void* emb_out, hipStream_t st) {
  size_t shm = sizeof(int32_t) * size_t(2 * K);
  int G = 64;
  while (G > 1 && G * K > kCbThreads) G >>= 1;
  const size_t total = size_t(B) * K * V;
  const uint16_t* E = static_cast<const uint16_t*>(cb_embed);
  uint16_t* out = static_cast<uint16_t*>(emb_out);
  if (f32)
    codebook_step_kernel<true><<<B, kCbThreads, shm, st>>>(K, V, G, bos, eoc, logits, total, frame, eoc_seen,
                                                           done, codes, aligned, max_frames, E, D, out);
  else
    codebook_step_kernel<false><<<B, kCbThreads, shm, st>>>(K, V, G, bos, eoc, logits, total, frame, eoc_seen,
                                                            done, codes, aligned, max_frames, E, D, out);
}

}  // namespace hr
