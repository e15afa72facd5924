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

// emb[b] = bf16( ((E[c0] + E[V+c1]) + ...) + E[(K-1)V + c_{K-1}] ), fp32 sum in
// codebook order; one 16-byte chunk of D per thread, the K rows loaded in
// batches of 8 before they are added
__device__ __forceinline__ void embed_sum(int b, int K, int V, const int32_t* s_code,
                                          const uint16_t* __restrict__ cb_embed, int D,
                                          uint16_t* __restrict__ emb_out) {
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

  embed_sum(b, K, V, s_code, cb_embed, D, emb_out);
}

// ====================================================== sampling + policies
// The step with per-stream sampling (vLLM-Omni pull request 8226, Higgs Audio v3
// streaming on Model Runner V2, Purpose and Test Plan: temperature, top-k and
// top-p with per-request seeded exponential noise) and the termination policies
// (FlashRT pull request 141, Summary and Root cause: delayed EOC for every
// codebook, a deterministic stop guard for repeated-code loops).
//
// One wavefront per codebook row; lane l holds the quads q = l + 64 j (elements
// 4q .. 4q+3) in registers, all loaded before any compare.  Integer keys that
// order like the logits (sign-folded bit patterns) make the top-k threshold and
// the top-p order exact: both thresholds are found bit by bit from the top,
// each probe a count (ballots) or a probability mass over the wave.  Masses
// are summed in a fixed order (per lane over its quads, then the DPP reduction
// below) and read from one lane, so the decisions are uniform over the wave.  The race draws Philox4x64-10 (Salmon et al.,
// SC 2011) for block (step, k, q, 0) under key (seed, 0): one block per quad,
// word w for element 4q + w.

constexpr uint64_t kPhM0 = 0xD2E7470EE14C6C93ull, kPhM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhW0 = 0x9E3779B97F4A7C15ull, kPhW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += kPhW0; k1 += kPhW1; }
    const uint64_t hi0 = __umul64hi(kPhM0, c[0]), lo0 = kPhM0 * c[0];
    const uint64_t hi1 = __umul64hi(kPhM1, c[2]), lo1 = kPhM1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

// u = (top 23 bits + 1/2) / 2^23: exact in binary32, inside (0, 1)
__device__ __forceinline__ float uniform23(uint64_t w) {
  return (float(uint32_t(w >> 41)) + 0.5f) * 1.1920928955078125e-7f;
}

// order-preserving key of a float (+0 and -0 share one key); 0 marks padding
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave reductions without a chain of LDS-pipe shuffles: DPP moves within rows
// of 16 lanes (quad swaps, half-row and row mirrors), then the row broadcasts
// of lanes 15 and 31 fold the four rows into lane 63, which every lane reads.
// The order of the additions is fixed, so every row gets the same rounding and
// every lane the same value.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_or(float x, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), CTRL, ROW_MASK, 0xf,
                                                    false));
}
__device__ __forceinline__ float wave_sum_u(float v) {
  v += dpp_or<0xb1>(v, 0.f);          // quad_perm(1, 0, 3, 2)
  v += dpp_or<0x4e>(v, 0.f);          // quad_perm(2, 3, 0, 1)
  v += dpp_or<0x141>(v, 0.f);         // row_half_mirror
  v += dpp_or<0x140>(v, 0.f);         // row_mirror: each row holds its sum
  v += dpp_or<0x142, 0xa>(v, 0.f);    // row_bcast:15 into rows 1 and 3
  v += dpp_or<0x143, 0xc>(v, 0.f);    // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max_u(float v) {
  const float ninf = -__builtin_inff();
  v = fmaxf(v, dpp_or<0xb1>(v, ninf));
  v = fmaxf(v, dpp_or<0x4e>(v, ninf));
  v = fmaxf(v, dpp_or<0x141>(v, ninf));
  v = fmaxf(v, dpp_or<0x140>(v, ninf));
  v = fmaxf(v, dpp_or<0x142, 0xa>(v, ninf));
  v = fmaxf(v, dpp_or<0x143, 0xc>(v, ninf));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

struct RowPolicy {
  float temperature;   // <= 0: greedy
  int top_k;           // <= 0 or >= V: off
  float top_p;         // >= 1: off; <= 0: the first element only
  uint64_t seed;
  int step, k;
};

// The same choice once at most 64 elements survive top-k: lane r holds the
// r-th survivor in index order (cx: logit, ck: key, cv: id; n survivors), so
// the top-p probes and the race cost one element per lane.
template <int KB>
__device__ int choose_compact(const float* cx, const uint32_t* ck, const int* cv, int n, const RowPolicy& P) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool valid = lane < n;
  uint32_t key = valid ? ck[lane] : 0u;
  const int v = valid ? cv[lane] : 0x7FFFFFFF;
  const float z = valid ? cx[lane] / P.temperature : 0.f;
  const float zmax = wave_max_u(valid ? z : -__builtin_inff());
  const float q = valid ? expf(z - zmax) : 0.f;
  const uint64_t lower = (1ull << lane) - 1ull;
  if (P.top_p < 1.f) {
    if (!(P.top_p > 0.f)) {
      // the first element of the order: the largest key, lowest index (lane)
      uint32_t km = key;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) km = max(km, uint32_t(__shfl_xor(km, m, kWave)));
      const uint64_t at = __ballot(key == km && valid);
      if (lane != __ffsll((unsigned long long)at) - 1) key = 0u;
    } else {
      const float pS = P.top_p * wave_sum_u(q);
      uint32_t vt = 0;
#pragma unroll 2
      for (int bit = KB - 1; bit >= 0; --bit) {
        const uint32_t cand = vt | (1u << bit);
        if (wave_sum_u(key >= cand ? q : 0.f) >= pS) vt = cand;
      }
      const float above = vt == (0xFFFFFFFFu >> (32 - KB)) ? 0.f : wave_sum_u(key > vt ? q : 0.f);
      const uint64_t ties = __ballot(key == vt);
      const float qt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(q), __ffsll((unsigned long long)ties) - 1));
      if (key < vt) key = 0u;
      else if (key == vt && !(above + float(__popcll(ties & lower)) * qt < pS)) key = 0u;
    }
  }
  float best = -__builtin_inff();
  int bi = 0x7FFFFFFF;
  if (key) {
    uint64_t c[4] = {uint64_t(uint32_t(P.step)), uint64_t(uint32_t(P.k)), uint64_t(v >> 2), 0ull};
    philox4x64_10(c, P.seed, 0ull);
    const uint64_t wv = (v & 3) == 0 ? c[0] : (v & 3) == 1 ? c[1] : (v & 3) == 2 ? c[2] : c[3];
    best = z - logf(-logf(uniform23(wv)));
    bi = v;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ob = __shfl_xor(best, m, kWave);
    const int oi = __shfl_xor(bi, m, kWave);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  return bi;
}

// Choice of one row by one wavefront (MQ quads per lane at most).  key[j][w]
// doubles as the membership of the element: 0 once it is out (padding, below
// the top-k threshold, past the top-p prefix).
template <bool F32, int MQ>
__device__ int choose_row(const void* __restrict__ logits, size_t row0, int V, const RowPolicy& P,
                          float* cx, uint32_t* cx_key, int* cx_id) {
  // keys: the order key of the logit; for bf16 logits its low half is
  // constant per sign, so the top 16 bits order them and the searches below
  // take 16 steps instead of 32
  constexpr int KB = F32 ? 32 : 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int nq = (V + 3) >> 2;
  float x[MQ][4];
  uint32_t key[MQ][4];
  // a quad is read as two pairs (4-byte bf16 / 8-byte fp32 loads) when the row
  // starts on an even element; a pair that runs past the row is read element
  // by element
  const bool pairs = (row0 & 1) == 0;
#pragma unroll
  for (int j = 0; j < MQ; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = 4 * (lane + kWave * j) + 2 * h;
      float f0 = -__builtin_inff(), f1 = -__builtin_inff();
      if (pairs && v + 1 < V) {
        if (F32) {
          const float2 t = *reinterpret_cast<const float2*>(static_cast<const float*>(logits) + row0 + v);
          f0 = t.x;
          f1 = t.y;
        } else {
          const uint32_t t = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(logits) + row0 + v);
          f0 = __uint_as_float(t << 16);
          f1 = __uint_as_float(t & 0xFFFF0000u);
        }
      } else {
        if (v < V) f0 = F32 ? static_cast<const float*>(logits)[row0 + v]
                            : __uint_as_float(uint32_t(static_cast<const uint16_t*>(logits)[row0 + v]) << 16);
        if (v + 1 < V) f1 = F32 ? static_cast<const float*>(logits)[row0 + v + 1]
                                : __uint_as_float(uint32_t(static_cast<const uint16_t*>(logits)[row0 + v + 1]) << 16);
      }
      x[j][2 * h] = f0;
      x[j][2 * h + 1] = f1;
      key[j][2 * h] = v < V ? order_key(f0) >> (32 - KB) : 0u;
      key[j][2 * h + 1] = v + 1 < V ? order_key(f1) >> (32 - KB) : 0u;
    }

  // largest key, lowest index among equals
  auto first_max = [&]() {
    uint32_t bk = 0;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < MQ; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (key[j][w] > bk) { bk = key[j][w]; bi = 4 * (lane + kWave * j) + w; }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const uint32_t ok = __shfl_xor(bk, m, kWave);
      const int oi = __shfl_xor(bi, m, kWave);
      if (ok > bk || (ok == bk && oi < bi)) { bk = ok; bi = oi; }
    }
    return bi;
  };
  if (!(P.temperature > 0.f)) return first_max();

  // top-k: the k-th largest key, found bit by bit (largest t with count(key >= t) >= k)
  if (P.top_k > 0 && P.top_k < V) {
    uint32_t thr = 0;
#pragma unroll 2
    for (int bit = KB - 1; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int n = 0;
#pragma unroll
      for (int j = 0; j < MQ; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) n += __popcll(__ballot(key[j][w] >= cand));
      if (n >= P.top_k) thr = cand;
    }
    int n_in = 0;
#pragma unroll
    for (int j = 0; j < MQ; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        key[j][w] = key[j][w] >= thr ? key[j][w] : 0u;
        n_in += __popcll(__ballot(key[j][w] != 0u));
      }
    if (n_in <= kWave) {
      // compact the survivors in index order: element (j, lane, w) follows
      // those of lower j, then of lower lanes, then of lower w
      const uint64_t lower = (1ull << lane) - 1ull;
      int before = 0;
#pragma unroll
      for (int j = 0; j < MQ; ++j) {
        int below = 0, total = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint64_t bw = __ballot(key[j][w] != 0u);
          below += __popcll(bw & lower);
          total += __popcll(bw);
        }
        int slot = before + below;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          if (key[j][w]) {
            cx[slot] = x[j][w];
            cx_key[slot] = key[j][w];
            cx_id[slot] = 4 * (lane + kWave * j) + w;
            ++slot;
          }
        before += total;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      return choose_compact<KB>(cx, cx_key, cx_id, n_in, P);
    }
  }

  // tempered logits and their softmax weights over the survivors
  float zmax = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < MQ; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[j][w] = x[j][w] / P.temperature;
      if (key[j][w]) zmax = fmaxf(zmax, x[j][w]);
    }
  zmax = wave_max_u(zmax);
  float q[MQ][4];
#pragma unroll
  for (int j = 0; j < MQ; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) q[j][w] = key[j][w] ? expf(x[j][w] - zmax) : 0.f;

  if (P.top_p < 1.f) {
    if (!(P.top_p > 0.f)) return first_max();
    auto mass_at_least = [&](uint32_t t) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < MQ; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) s += key[j][w] >= t ? q[j][w] : 0.f;
      return wave_sum_u(s);
    };
    const float pS = P.top_p * mass_at_least(1u);
    // the crossing key: largest t with mass(key >= t) >= p S
    uint32_t vt = 0;
#pragma unroll 2
    for (int bit = KB - 1; bit >= 0; --bit) {
      const uint32_t cand = vt | (1u << bit);
      if (mass_at_least(cand) >= pS) vt = cand;
    }
    const float above = vt == (0xFFFFFFFFu >> (32 - KB)) ? 0.f : mass_at_least(vt + 1u);
    // elements with key == vt are equal: each is kept while the mass ahead of
    // it (above + the equal ones of lower index) stays below p S
    float qt = 0.f;
#pragma unroll
    for (int j = 0; j < MQ; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (key[j][w] == vt) qt = q[j][w];
    int before = 0;   // equal elements in the quads of lower j
    const uint64_t lower = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < MQ; ++j) {
      int lanes_below = 0, total = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint64_t bw = __ballot(key[j][w] == vt);
        lanes_below += __popcll(bw & lower);
        total += __popcll(bw);
      }
      int here = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (key[j][w] == vt) {
          if (!(above + float(before + lanes_below + here) * qt < pS)) key[j][w] = 0u;
          ++here;
        } else if (key[j][w] < vt) {
          key[j][w] = 0u;
        }
      }
      before += total;
    }
  }

  // exponential race: largest z - ln(-ln u) over the kept elements (a row
  // with no comparable score, e.g. NaN logits, falls back to its argmax so the
  // code is always an id of the row)
  float best = -__builtin_inff();
  int bi = 0x7FFFFFFF;
#pragma unroll
  for (int j = 0; j < MQ; ++j) {
    const int qd = lane + kWave * j;
    const bool any = (key[j][0] | key[j][1] | key[j][2] | key[j][3]) != 0u;
    if (__ballot(any) == 0) continue;
    uint64_t c[4] = {uint64_t(uint32_t(P.step)), uint64_t(uint32_t(P.k)), uint64_t(qd), 0ull};
    if (qd < nq) philox4x64_10(c, P.seed, 0ull);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (!key[j][w]) continue;
      const float e = -logf(uniform23(c[w]));
      const float sc = x[j][w] - logf(e);
      const int v = 4 * qd + w;
      if (sc > best || (sc == best && v < bi)) { best = sc; bi = v; }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ob = __shfl_xor(best, m, kWave);
    const int oi = __shfl_xor(bi, m, kWave);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  return bi < V ? bi : first_max();
}

template <bool F32, int MQ>
__global__ __launch_bounds__(kCbThreads) void codebook_policy_kernel(
    int K, int V, int bos, int eoc, const void* __restrict__ logits,
    int32_t* __restrict__ frame, uint8_t* __restrict__ eoc_seen, uint8_t* __restrict__ done,
    int32_t* __restrict__ codes, int32_t* __restrict__ aligned, int max_frames,
    const uint16_t* __restrict__ cb_embed, int D, uint16_t* __restrict__ emb_out, StepPolicy pol) {
  // [K] choices, then codes; [K, 2K) seen flags; then per wave 64 compacted
  // survivors (logit, key, id)
  extern __shared__ int32_t s_code[];
  const int b = blockIdx.x;
  const bool is_done = done[b] != 0;
  const int t = frame[b];
  const int e = pol.end_frame ? pol.end_frame[b] : -1;
  int32_t* s_wave = s_code + 2 * K + (threadIdx.x / kWave) * 3 * kWave;
  RowPolicy P;
  P.temperature = pol.temperature ? pol.temperature[b] : 0.f;
  P.top_k = pol.top_k ? pol.top_k[b] : 0;
  P.top_p = pol.top_p ? pol.top_p[b] : 1.f;
  P.seed = pol.seed ? pol.seed[b] : 0ull;
  P.step = t;
  for (int k = threadIdx.x; k < K; k += blockDim.x) s_code[K + k] = eoc_seen[size_t(b) * K + k];
  __syncthreads();

  if (!is_done) {
    const int wave = threadIdx.x / kWave;
    for (int k = wave; k < K; k += kCbThreads / kWave) {
      // rows whose code is fixed (delay fill, sticky or forced EOC) need no choice
      if (t < k || s_code[K + k] != 0 || (e >= 0 && t >= e + k)) continue;
      P.k = k;
      const int r = choose_row<F32, MQ>(logits, (size_t(b) * K + k) * V, V, P, reinterpret_cast<float*>(s_wave),
                                        reinterpret_cast<uint32_t*>(s_wave + kWave), s_wave + 2 * kWave);
      if ((threadIdx.x & (kWave - 1)) == 0) s_code[k] = (r >= 0 && r < V) ? r : 0;
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    int c = eoc;
    if (!is_done) {
      const bool seen = s_code[K + k] != 0;
      c = (t < k) ? bos : (seen || (e >= 0 && t >= e + k)) ? eoc : s_code[k];
      if (c == eoc && !seen) eoc_seen[size_t(b) * K + k] = 1;
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
    if (e < 0) {
      int cand = 0x7FFFFFFF;
      if (pol.repeat_limit > 0) {
        int32_t* last = pol.last_codes + size_t(b) * K;
        bool same = true;
        for (int k = 0; k < K; ++k) {
          same = same && last[k] == s_code[k];
          last[k] = s_code[k];
        }
        const int run = same ? pol.repeat_run[b] + 1 : 1;
        pol.repeat_run[b] = run;
        if (run >= pol.repeat_limit) cand = t + 1;
      }
      if (pol.eoc_cascade) {
        int kmax = -1;
        for (int k = 0; k < K; ++k)
          if (s_code[k] == eoc) kmax = k;
        if (kmax >= 0) cand = min(cand, t - kmax);
      }
      if (cand != 0x7FFFFFFF) pol.end_frame[b] = cand;
    }
    frame[b] = t + 1;
    done[b] = all ? 1 : 0;
  }

  embed_sum(b, K, V, s_code, cb_embed, D, emb_out);
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

void launch_codebook_policy(int B, int K, int V, int bos, int eoc, bool f32, const void* logits,
                            int32_t* frame, uint8_t* eoc_seen, uint8_t* done, int32_t* codes,
                            int32_t* aligned, int max_frames, const void* cb_embed, int D,
                            void* emb_out, const StepPolicy& pol, hipStream_t st) {
  const size_t shm = sizeof(int32_t) * (size_t(2 * K) + (kCbThreads / kWave) * 3 * kWave);
  const uint16_t* E = static_cast<const uint16_t*>(cb_embed);
  uint16_t* out = static_cast<uint16_t*>(emb_out);
#define HR_POLICY(F, MQ)                                                                          \
  codebook_policy_kernel<F, MQ><<<B, kCbThreads, shm, st>>>(K, V, bos, eoc, logits, frame, eoc_seen, \
                                                             done, codes, aligned, max_frames, E, D,  \
                                                             out, pol)
  const int nq = (V + 3) / 4;
  if (f32) {
    if (nq <= 2 * kWave) HR_POLICY(true, 2);
    else if (nq <= 5 * kWave) HR_POLICY(true, 5);
    else HR_POLICY(true, 8);
  } else {
    if (nq <= 2 * kWave) HR_POLICY(false, 2);
    else if (nq <= 5 * kWave) HR_POLICY(false, 5);
    else HR_POLICY(false, 8);
  }
#undef HR_POLICY
}

}  // namespace hr
