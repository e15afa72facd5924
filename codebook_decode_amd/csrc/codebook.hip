// Delayed-codebook step (FlashRT pull request 141 "Stabilize Higgs Audio
// termination and prefill", Summary and Root cause): per-frame argmax of every
// codebook, delay-pattern bookkeeping (BOS fill while t < k, sticky per-codebook
// EOC, done once every codebook has emitted EOC) and the codebook-embedding sum
// that feeds the next decode step.
//
// One workgroup per stream, 256 threads.  Each wavefront takes codebooks
// w, w+4, ...: lanes scan strided ids and keep (max, lowest index), then a
// butterfly reduction picks the row's first maximum.  Lane k applies codebook
// k's delay / EOC update; one lane then updates the frame counter and done.
// The workgroup then sums the K selected embedding rows with 128-bit loads,
// in codebook order, in fp32, and rounds once to bf16.
#include "common.h"
#include "launch.h"

namespace hr {

template <bool F32>
__device__ __forceinline__ float logit_at(const void* p, size_t i) {
  if (F32) return static_cast<const float*>(p)[i];
  return bf2f(static_cast<const uint16_t*>(p)[i]);
}

template <bool F32>
__global__ __launch_bounds__(256) void codebook_step_kernel(
    int K, int V, int bos, int eoc, const void* __restrict__ logits, int32_t* __restrict__ frame,
    uint8_t* __restrict__ eoc_seen, uint8_t* __restrict__ done, int32_t* __restrict__ codes,
    int32_t* __restrict__ aligned, int max_frames, const uint16_t* __restrict__ cb_embed, int D,
    uint16_t* __restrict__ emb_out) {
  extern __shared__ int32_t s_code[];  // [K] argmax ids, then chosen codes; [K, 2K) seen flags
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool is_done = done[b] != 0;

  if (!is_done) {
    for (int k = wave; k < K; k += 4) {
      size_t row = (size_t(b) * K + k) * V;
      float best = -__builtin_inff();
      int bi = 0x7FFFFFFF;
      for (int v = lane; v < V; v += 64) {
        float x = logit_at<F32>(logits, row + v);
        if (x > best || bi == 0x7FFFFFFF) { best = x; bi = v; }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        float ob = __shfl_xor(best, m, kWave);
        int oi = __shfl_xor(bi, m, kWave);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      if (lane == 0) s_code[k] = bi;
    }
  }
  __syncthreads();
  // delay / EOC bookkeeping: one lane per codebook, then one lane for the stream
  const int t = frame[b];
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    int c = eoc;
    if (!is_done) {
      const size_t ks = size_t(b) * K + k;
      uint8_t seen = eoc_seen[ks];
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
    const u32x4* r0 = reinterpret_cast<const u32x4*>(cb_embed + size_t(s_code[0]) * D) + d8;
    u32x4 w = *r0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { acc[2 * j] = bf_lo(w[j]); acc[2 * j + 1] = bf_hi(w[j]); }
    for (int k = 1; k < K; ++k) {
      const u32x4* rk = reinterpret_cast<const u32x4*>(cb_embed + (size_t(k) * V + s_code[k]) * D) + d8;
      u32x4 x = *rk;
#pragma unroll
      for (int j = 0; j < 4; ++j) { acc[2 * j] += bf_lo(x[j]); acc[2 * j + 1] += bf_hi(x[j]); }
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
  const uint16_t* E = static_cast<const uint16_t*>(cb_embed);
  uint16_t* out = static_cast<uint16_t*>(emb_out);
  if (f32)
    codebook_step_kernel<true><<<B, 256, shm, st>>>(K, V, bos, eoc, logits, frame, eoc_seen, done,
                                                    codes, aligned, max_frames, E, D, out);
  else
    codebook_step_kernel<false><<<B, 256, shm, st>>>(K, V, bos, eoc, logits, frame, eoc_seen, done,
                                                     codes, aligned, max_frames, E, D, out);
}

}  // namespace hr
