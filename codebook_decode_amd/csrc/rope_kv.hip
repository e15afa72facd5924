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
// 32-byte pieces straight from the fp32 merged QKV row (the d/16 lanes of a
// row read 4 x d bytes, whole 128-byte lines), the head's sum of squares is a
// butterfly over those lanes, and the results leave as 16-byte stores: q in
// fp16, k and v in bf16 (the cache), each value rounded once.  Rows are dealt
// to the threads in rounds of 256 / (d/16), kRopeRows rounds in flight.
#include <cmath>

#include "common.h"
#include "launch.h"
#include "rope_math.h"

namespace hr {

constexpr int kRopeTok = 4;     // tokens per workgroup
constexpr int kRopeRows = 3;    // head-row rounds with loads in flight per thread

__global__ __launch_bounds__(256) void qknorm_rope_kv_kernel(
    const float* __restrict__ qkv, int T, int tpb, int Hq, int Hkv, int d, const RopeFreq freq, float eps,
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
  F8 lo[kRopeRows], hi[kRopeRows];
  auto load_round = [&](int base) {
#pragma unroll
    for (int k = 0; k < kRopeRows; ++k) {
      const int rr = base + k * per_round;
      if (rr < total) {
        const int tt = rr / n_rows, r = rr % n_rows;
        const float* src = qkv + size_t(t0 + tt) * n_rows * d + size_t(r) * d;
        lo[k] = load_f8(src + 8 * c);
        hi[k] = load_f8(src + half + 8 * c);
      } else {
        lo[k] = F8{floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
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
    rope_angle(p, freq.inv[m], s_cos[tt][m], s_sin[tt][m]);
  }
  __syncthreads();

  for (; base < total; base += step) {
    if (base != tid / L) load_round(base);
#pragma unroll
    for (int k = 0; k < kRopeRows; ++k) {
      const int rr = base + k * per_round;
      const float ss = group_sum(pairs_sumsq(lo[k], hi[k]), L);   // every lane of the wave takes part
      if (rr >= total) continue;
      const int tt = rr / n_rows, r = rr % n_rows;
      const int t = t0 + tt;
      if (r < Hq + Hkv) {
        const bool is_q = r < Hq;
        if (!is_q && !s_wkv[tt]) continue;
        const float inv = 1.0f / __builtin_sqrtf(ss / float(d) + eps);
        F8 o0, o1;
        rope_pairs(lo[k], hi[k], is_q ? wq0 : wk0, is_q ? wq1 : wk1, inv, &s_cos[tt][8 * c], &s_sin[tt][8 * c],
                   o0, o1);
        uint16_t* dst = is_q ? q_out + (size_t(t) * Hq + r) * d
                             : kc + (size_t(s_crow[tt]) * Hkv + (r - Hq)) * d;
        *reinterpret_cast<u32x4*>(dst + 8 * c) = is_q ? pack8_f16(o0) : pack8_bf16(o0);
        *reinterpret_cast<u32x4*>(dst + half + 8 * c) = is_q ? pack8_f16(o1) : pack8_bf16(o1);
      } else if (s_wkv[tt]) {
        uint16_t* dst = vc + (size_t(s_crow[tt]) * Hkv + (r - Hq - Hkv)) * d;
        *reinterpret_cast<u32x4*>(dst + 8 * c) = pack8_bf16(lo[k]);
        *reinterpret_cast<u32x4*>(dst + half + 8 * c) = pack8_bf16(hi[k]);
      }
    }
  }
}

// The angle table of a batch for the QKV epilogue (launch_qkv_rope): one
// thread per (token, pair m), the same angle arithmetic as the table of
// qknorm_rope_kv_kernel, so both paths rotate by the same bits.
__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t* __restrict__ cu,
                                                         const int32_t* __restrict__ start_pos, int n_seq, int T,
                                                         int half, const RopeFreq freq, float* __restrict__ tab) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * half) return;
  const int t = idx / half, m = idx % half;
  const int s = find_seq(cu, n_seq, t);
  const int p = start_pos[s] + (t - cu[s]);
  float cs, sn;
  rope_angle(p, freq.inv[m], cs, sn);
  tab[size_t(t) * 2 * half + m] = cs;
  tab[size_t(t) * 2 * half + half + m] = sn;
}

void launch_rope_table(const int32_t* cu, const int32_t* start_pos, int n_seq, int T, int d, float theta,
                       float* tab, hipStream_t st) {
  const int half = d / 2;
  const RopeFreq freq = rope_freq(d, theta);
  rope_table_kernel<<<(T * half + 255) / 256, 256, 0, st>>>(cu, start_pos, n_seq, T, half, freq, tab);
}

void launch_qknorm_rope_kv(const void* qkv, int T, int Hq, int Hkv, int d, float theta, float eps,
                           const int32_t* cu, const int32_t* start_pos, const int32_t* cache_slot,
                           const int32_t* used_keys, int n_seq, bool causal, const void* qw,
                           const void* kw, void* q_out, void* kc, void* vc, int capacity,
                           hipStream_t st) {
  // tokens per workgroup: 1 up to 2048 tokens (latency: every row in flight
  // at once; T = 512: 6.9 us against 7.6 with 2, T = 1024: 8.9 against 12.3),
  // kRopeTok for large batches (fewer angle tables; T = 4096: 22.6 us against
  // 26.1 with 1)
  const int tpb = T <= 2048 ? 1 : (T < 4096 ? 2 : kRopeTok);
  const int blocks = (T + tpb - 1) / tpb;
  const RopeFreq freq = rope_freq(d, theta);
  qknorm_rope_kv_kernel<<<blocks, 256, 0, st>>>(
      static_cast<const float*>(qkv), T, tpb, Hq, Hkv, d, freq, eps, cu, start_pos, cache_slot,
      used_keys, n_seq, causal ? 1 : 0, static_cast<const uint16_t*>(qw),
      static_cast<const uint16_t*>(kw), static_cast<uint16_t*>(q_out), static_cast<uint16_t*>(kc),
      static_cast<uint16_t*>(vc), capacity);
}

// ======================================================= short prompts: steps A3 + A4
// A prompt of at most kSmallRows rows that starts at position 0 attends to its
// own rows only, so one workgroup per (query head, sequence) can norm and
// rotate the rows it needs (its q head, and the k and v heads of its group),
// write K and V to the cache (the group's first query head does), and run the
// softmax from LDS, which saves the round trip of q through memory and a
// launch whose work is tiny at these sizes.  The rows get the same arithmetic
// as in qknorm_rope_kv_kernel (pairs_sumsq, rope_pairs, rope_angle), so the
// cache receives the same bits.  8 waves; wave w takes queries w, w + 8, ...
// (NQ of them, the last ones clamped and discarded, so that no loop branches).
// Scores: lane j takes key j; the k rows sit in LDS padded by 16 bytes (one
// 16-byte read per lane and d step, no bank conflict), q rows are broadcast
// reads.  Softmax in fp32 (base 2, the scale folded into one multiply) with the
// exact row max; the max and the sum are DPP reductions within rows of 16
// lanes and a fixed-order combination of the 4 rows.  P V: lane l owns output
// dims 2l and 2l + 1 and takes each probability from lane j by readlane.  The
// output is o / l rounded once (fp16, or e4m3 of o / l times out_inv).  q is
// held in fp16 and k, v in bf16, the values the separate kernels store.
// Causal: keys j <= i; otherwise keys j < used_keys[s].
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_f(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}
// max / sum over the wave: within each row of 16 lanes (quad swaps, then the
// half-row and row mirrors: every source lane exists), then over the 4 rows
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_row<0xb1>(v));
  v = fmaxf(v, dpp_row<0x4e>(v));
  v = fmaxf(v, dpp_row<0x141>(v));
  v = fmaxf(v, dpp_row<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = v + dpp_row<0xb1>(v);
  v = v + dpp_row<0x4e>(v);
  v = v + dpp_row<0x141>(v);
  v = v + dpp_row<0x140>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

constexpr int kSmallWaves = 8;

template <int D, int NQ>
__global__ __launch_bounds__(64 * kSmallWaves) void rope_attn_small_kernel(
    const float* __restrict__ qkv, int Hq, int Hkv, const RopeFreq freq, float eps,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cache_slot, const int32_t* __restrict__ used_keys,
    int causal, const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw, uint16_t* __restrict__ kc,
    uint16_t* __restrict__ vc, int capacity, float scale_log2, void* __restrict__ out, int out_fp8,
    float out_inv) {
  constexpr int NT = 64 * kSmallWaves;
  constexpr int HALF = D / 2, L = D / 16, PER = NT / L;     // lanes per head row, rows per round
  constexpr int NR = (3 * kSmallRows + PER - 1) / PER;      // rounds of rows (all loads in flight)
  constexpr int KLD = D + 8;                                 // padded k row (elements)
  __shared__ float s_cos[kSmallRows][HALF], s_sin[kSmallRows][HALF];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kSmallRows][D];
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kSmallRows][KLD];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kSmallRows][D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq = blockIdx.x, s = blockIdx.y;
  const int G = Hq / Hkv, g = hq / G;
  const int t0 = cu[s], len = cu[s + 1] - t0;
  if (len <= 0) return;                                      // whole workgroup: no barrier skipped
  const int n_keys = causal ? len : used_keys[s];
  const bool write_kv = hq % G == 0;
  const long long crow0 = (long long)cache_slot[s] * capacity;
  const int n_rows = Hq + 2 * Hkv;
  const int c = tid % L;

  // rows rr < 3 len: q of token rr, then k of token rr - len, then v
  F8 lo[NR], hi[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int rr = tid / L + k * PER;
    if (rr < 3 * len) {
      const int kind = rr / len, i = rr - kind * len;
      const int head = kind == 0 ? hq : (kind == 1 ? Hq + g : Hq + Hkv + g);
      const float* src = qkv + (size_t(t0 + i) * n_rows + head) * D;
      lo[k] = load_f8(src + 8 * c);
      hi[k] = load_f8(src + HALF + 8 * c);
    } else {
      lo[k] = F8{floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
      hi[k] = lo[k];
    }
  }
  const u32x4 wq0 = *reinterpret_cast<const u32x4*>(qw + 8 * c);
  const u32x4 wq1 = *reinterpret_cast<const u32x4*>(qw + HALF + 8 * c);
  const u32x4 wk0 = *reinterpret_cast<const u32x4*>(kw + 8 * c);
  const u32x4 wk1 = *reinterpret_cast<const u32x4*>(kw + HALF + 8 * c);
  for (int a = tid; a < len * HALF; a += NT) {
    const int i = a / HALF, m = a % HALF;
    rope_angle(i, freq.inv[m], s_cos[i][m], s_sin[i][m]);
  }
  __syncthreads();

#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int rr = tid / L + k * PER;
    const float ss = group_sum(pairs_sumsq(lo[k], hi[k]), L);   // every lane of the wave takes part
    if (rr >= 3 * len) continue;
    const int kind = rr / len, i = rr - kind * len;
    const bool kv_row = write_kv && (causal || i < n_keys);
    if (kind < 2) {
      const float inv = 1.0f / __builtin_sqrtf(ss / float(D) + eps);
      F8 r0, r1;
      rope_pairs(lo[k], hi[k], kind == 0 ? wq0 : wk0, kind == 0 ? wq1 : wk1, inv, &s_cos[i][8 * c],
                 &s_sin[i][8 * c], r0, r1);
      const u32x4 o0 = kind == 0 ? pack8_f16(r0) : pack8_bf16(r0);
      const u32x4 o1 = kind == 0 ? pack8_f16(r1) : pack8_bf16(r1);
      uint16_t* row = kind == 0 ? &s_q[i][0] : &s_k[i][0];
      *reinterpret_cast<u32x4*>(row + 8 * c) = o0;
      *reinterpret_cast<u32x4*>(row + HALF + 8 * c) = o1;
      if (kind == 1 && kv_row) {
        uint16_t* dst = kc + (size_t(crow0 + i) * Hkv + g) * D;
        *reinterpret_cast<u32x4*>(dst + 8 * c) = o0;
        *reinterpret_cast<u32x4*>(dst + HALF + 8 * c) = o1;
      }
    } else {
      const u32x4 v0 = pack8_bf16(lo[k]), v1 = pack8_bf16(hi[k]);
      *reinterpret_cast<u32x4*>(&s_v[i][8 * c]) = v0;
      *reinterpret_cast<u32x4*>(&s_v[i][HALF + 8 * c]) = v1;
      if (kv_row) {
        uint16_t* dst = vc + (size_t(crow0 + i) * Hkv + g) * D;
        *reinterpret_cast<u32x4*>(dst + 8 * c) = v0;
        *reinterpret_cast<u32x4*>(dst + HALF + 8 * c) = v1;
      }
    }
  }
  __syncthreads();
  if (wave >= len) return;                                   // no query for this wave (no barrier follows)

  // scores of queries i = wave + 8 qi (clamped to the last row) against key j = lane
  int qrow[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) qrow[qi] = min(wave + kSmallWaves * qi, len - 1);
  const int krow = lane < n_keys ? lane : n_keys - 1;
  float acc[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) acc[qi] = 0.f;
#pragma unroll 4
  for (int d8 = 0; d8 < D / 8; ++d8) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(&s_k[krow][8 * d8]);
    u32x4 qv[NQ];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) qv[qi] = *reinterpret_cast<const u32x4*>(&s_q[qrow[qi]][8 * d8]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float kf = bf_at(kv, e);
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) acc[qi] += h_at(qv[qi], e) * kf;
    }
  }
  float p[NQ], inv_l[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const int i = wave + kSmallWaves * qi;
    const bool ok = causal ? lane <= i : lane < n_keys;      // lane 0 always: the max is finite
    const float x = ok ? acc[qi] * scale_log2 : -INFINITY;
    const float mx = wave_max_dpp(x);
    p[qi] = ok ? exp2f(x - mx) : 0.f;
    inv_l[qi] = 1.0f / wave_sum_dpp(p[qi]);
  }

  // o = P V: lane l owns dims 2l, 2l + 1
  const int dl = lane < HALF ? lane : HALF - 1;
  float o0[NQ], o1[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) o0[qi] = o1[qi] = 0.f;
  const int j_end = causal ? min(len, wave + kSmallWaves * (NQ - 1) + 1) : n_keys;
#pragma unroll 4
  for (int j = 0; j < j_end; ++j) {
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(&s_v[j][2 * dl]);
    const float v0 = bf_lo(vv), v1 = bf_hi(vv);
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      const float pj = lane_f(p[qi], j);
      o0[qi] += pj * v0;
      o1[qi] += pj * v1;
    }
  }
  if (lane < HALF) {
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      const int i = wave + kSmallWaves * qi;
      if (i < len) {
        const float y0 = o0[qi] * inv_l[qi], y1 = o1[qi] * inv_l[qi];
        const size_t orow = (size_t(t0 + i) * Hq + hq) * D + 2 * lane;
        if (out_fp8)
          *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(out) + orow) =
              uint16_t(f2e4m3(y0 * out_inv) | (f2e4m3(y1 * out_inv) << 8));
        else
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + orow) = pack_f16x2(y0, y1);
      }
    }
  }
}

void launch_rope_attn_small(const void* qkv, int n_seq, int max_len, int Hq, int Hkv, int d, float theta, float eps,
                            const int32_t* cu, const int32_t* cache_slot, const int32_t* used_keys, bool causal,
                            const void* qw, const void* kw, void* kc, void* vc, int capacity, void* out, bool fp8,
                            float out_inv, hipStream_t st) {
  const RopeFreq freq = rope_freq(d, theta);
  const float scale_log2 = 1.4426950408889634f / __builtin_sqrtf(float(d));
  const dim3 grid(Hq, n_seq);
  auto go = [&](auto kern) {
    kern<<<grid, 64 * kSmallWaves, 0, st>>>(
        static_cast<const float*>(qkv), Hq, Hkv, freq, eps, cu, cache_slot, used_keys, causal ? 1 : 0,
        static_cast<const uint16_t*>(qw), static_cast<const uint16_t*>(kw), static_cast<uint16_t*>(kc),
        static_cast<uint16_t*>(vc), capacity, scale_log2, out, fp8 ? 1 : 0, out_inv);
  };
  // queries per wave: the longest sequence's rows over the 8 waves
  const int nq = (max_len + kSmallWaves - 1) / kSmallWaves;
  if (d == 128) {
    if (nq <= 1) go(rope_attn_small_kernel<128, 1>);
    else if (nq == 2) go(rope_attn_small_kernel<128, 2>);
    else go(rope_attn_small_kernel<128, 4>);
  } else {
    if (nq <= 1) go(rope_attn_small_kernel<64, 1>);
    else if (nq == 2) go(rope_attn_small_kernel<64, 2>);
    else go(rope_attn_small_kernel<64, 4>);
  }
}

}  // namespace hr
