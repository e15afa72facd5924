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
    const float* __restrict__ qkv, const int32_t* __restrict__ cu, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ cache_slot, const int32_t* __restrict__ used_keys, int T, int tpb, int Hq, int Hkv,
    int d, int n_seq, int causal, float eps, const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
    uint16_t* __restrict__ q_out, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int capacity,
    const RopeFreq freq) {   // the 512-byte table last: the pointers above fit the preloaded argument words
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
      static_cast<const float*>(qkv), cu, start_pos, cache_slot, used_keys, T, tpb, Hq, Hkv, d, n_seq,
      causal ? 1 : 0, eps, static_cast<const uint16_t*>(qw), static_cast<const uint16_t*>(kw),
      static_cast<uint16_t*>(q_out), static_cast<uint16_t*>(kc), static_cast<uint16_t*>(vc), capacity, freq);
}

// ======================================================= short prompts: steps A3 + A4
// A prompt of at most kSmallRows rows that starts at position 0 attends to its
// own rows only, so one workgroup per (query head, sequence) can norm and
// rotate the rows it needs (its q head, and the k and v heads of its group),
// write K and V to the cache (the group's first query head does), and run the
// softmax from LDS, which saves the round trip of q through memory and a
// launch whose work is tiny at these sizes.  The rows get the same arithmetic
// as in qknorm_rope_kv_kernel (pairs_sumsq, rope_pairs, rope_angle), so the
// cache receives the same bits.  8 waves share the row work (a wave takes
// rows of one kind); then one wave computes the head's attention as one block
// of 32 queries x 32 keys with v_mfma_f32_32x32x16_f16, in the form of
// attention_kernel: S^T = K Q^T (the
// lane's accumulator column is query l % 32, its 16 rows keys
// 8(r/4) + 4(l/32) + r%4), the softmax per lane plus one exchange with lane
// l ^ 32, then O^T = V^T P^T with the lane's own probabilities as the B
// operand.  LDS holds q in fp16 (as the separate q/k-norm kernel stores it),
// k and v as their bf16 cache values widened exactly to fp16, v transposed
// (its columns past the prompt zero, so masked keys add 0 x 0).  Rows past the
// prompt read its last row (finite; their scores are masked or their outputs
// not stored).  Softmax in fp32, base 2 with the scale folded into one FMA,
// probabilities rounded to fp16 for the MFMA; the output is o / l rounded once
// (fp16, or e4m3 of o / l times out_inv).
// Causal: keys j <= i; otherwise keys j < used_keys[s].
constexpr int kSmallWaves = 8;

__device__ __forceinline__ floatx16 mfma32x16_f16(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

template <int D>
__global__ __launch_bounds__(64 * kSmallWaves) void rope_attn_small_kernel(
    const float* __restrict__ qkv, const int32_t* __restrict__ cu, const int32_t* __restrict__ cache_slot,
    const int32_t* __restrict__ used_keys, int Hq, int Hkv, int causal, float eps, const uint16_t* __restrict__ qw,
    const uint16_t* __restrict__ kw, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int capacity,
    float scale_log2, void* __restrict__ out, int out_fp8, float out_inv, const float* __restrict__ tab,
    const RopeFreq freq) {   // the 512-byte table last: the pointers above fit the preloaded argument words
  static_assert(kSmallRows == 32, "one 32 x 32 block of queries and keys");
  constexpr int NT = 64 * kSmallWaves;
  constexpr int HALF = D / 2, L = D / 16, RPW = kWave / L;  // lanes per head row, rows per wave
  // rounds of head rows (all loads in flight): a wave takes RPW rows of one
  // kind (q, k or v), ceil(len / RPW) waves per kind, so no wave branches on
  // the kind and the three kinds run side by side
  constexpr int NR = (3 * ((kSmallRows + RPW - 1) / RPW) + kSmallWaves - 1) / kSmallWaves;
  constexpr int LD = D + 8;                                  // padded q / k row (elements)
  // key stride of v^T: 17 words, odd, so the 32 rows of a fragment read and
  // the rows 8c + 2e that a v row's 8 lanes scatter to fall in distinct banks
  constexpr int VLD = kSmallRows + 2;
  constexpr int NKS = D / 16, NDB = D / 32;
  __shared__ float s_cos[kSmallRows][HALF], s_sin[kSmallRows][HALF];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kSmallRows][LD];
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kSmallRows][LD];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[D][VLD];
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
  const int kw_waves = (len + RPW - 1) / RPW;                // waves per kind

  // round k of wave w is slot w' = 8 k + w: kind w' / kw_waves (0 q, 1 k, 2 v),
  // row RPW (w' % kw_waves) + lane / L of that kind
  F8 lo[NR], hi[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int slot = k * kSmallWaves + wave, kind = slot / kw_waves;
    const int i = (slot % kw_waves) * RPW + lane / L;
    if (kind < 3 && i < len) {
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
  if (!tab) {                                                 // else the batch's table (rope_table_kernel)
    for (int a = tid; a < len * HALF; a += NT) {
      const int i = a / HALF, m = a % HALF;
      rope_angle(i, freq.inv[m], s_cos[i][m], s_sin[i][m]);
    }
  }
  // v^T zeroed (the columns past the prompt stay zero: their probabilities are 0)
  for (int a = tid; a < D * (kSmallRows / 2); a += NT)
    reinterpret_cast<uint32_t*>(&s_vt[0][0])[(a / (kSmallRows / 2)) * (VLD / 2) + a % (kSmallRows / 2)] = 0u;
  __syncthreads();

#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int slot = k * kSmallWaves + wave, kind = slot / kw_waves;
    const int i = (slot % kw_waves) * RPW + lane / L;
    const float ss = group_sum(pairs_sumsq(lo[k], hi[k]), L);   // every lane of the wave takes part
    if (kind >= 3 || i >= len) continue;
    const bool kv_row = write_kv && (causal || i < n_keys);
    if (kind < 2) {
      const float inv = 1.0f / __builtin_sqrtf(ss / float(D) + eps);
      F8 r0, r1;
      const float* cs = tab ? tab + size_t(t0 + i) * D + 8 * c : &s_cos[i][8 * c];
      const float* sn = tab ? cs + HALF : &s_sin[i][8 * c];
      rope_pairs(lo[k], hi[k], kind == 0 ? wq0 : wk0, kind == 0 ? wq1 : wk1, inv, cs, sn, r0, r1);
      if (kind == 0) {
        *reinterpret_cast<u32x4*>(&s_q[i][8 * c]) = pack8_f16(r0);
        *reinterpret_cast<u32x4*>(&s_q[i][HALF + 8 * c]) = pack8_f16(r1);
      } else {
        const u32x4 o0 = pack8_bf16(r0), o1 = pack8_bf16(r1);
        *reinterpret_cast<u32x4*>(&s_k[i][8 * c]) = bf8_to_f16x8(o0);
        *reinterpret_cast<u32x4*>(&s_k[i][HALF + 8 * c]) = bf8_to_f16x8(o1);
        if (kv_row) {
          uint16_t* dst = kc + (size_t(crow0 + i) * Hkv + g) * D;
          *reinterpret_cast<u32x4*>(dst + 8 * c) = o0;
          *reinterpret_cast<u32x4*>(dst + HALF + 8 * c) = o1;
        }
      }
    } else {
      const u32x4 v0 = pack8_bf16(lo[k]), v1 = pack8_bf16(hi[k]);
      const u32x4 h0 = bf8_to_f16x8(v0), h1 = bf8_to_f16x8(v1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_vt[8 * c + 2 * e][i] = uint16_t(h0[e]);
        s_vt[8 * c + 2 * e + 1][i] = uint16_t(h0[e] >> 16);
        s_vt[HALF + 8 * c + 2 * e][i] = uint16_t(h1[e]);
        s_vt[HALF + 8 * c + 2 * e + 1][i] = uint16_t(h1[e] >> 16);
      }
      if (kv_row) {
        uint16_t* dst = vc + (size_t(crow0 + i) * Hkv + g) * D;
        *reinterpret_cast<u32x4*>(dst + 8 * c) = v0;
        *reinterpret_cast<u32x4*>(dst + HALF + 8 * c) = v1;
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;                                     // one wave per head (no barrier follows)

  const int half = lane >> 5, r32 = lane & 31;
  const int qrow = min(r32, len - 1), krow = qrow;           // rows past the prompt: its last row
  floatx16 sc;
#pragma unroll
  for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const u32x4 kf = *reinterpret_cast<const u32x4*>(&s_k[krow][16 * ks + 8 * half]);
    const u32x4 qf = *reinterpret_cast<const u32x4*>(&s_q[qrow][16 * ks + 8 * half]);
    sc = mfma32x16_f16(kf, qf, sc);
  }
  // lane: query j = r32; element r: key 8(r/4) + 4 half + r%4
  const int j_max = causal ? r32 : n_keys - 1;
  float mt = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 8 * (r >> 2) + 4 * half + (r & 3);
    if (key > j_max) sc[r] = -INFINITY;
    mt = fmaxf(mt, sc[r]);
  }
  mt = fmaxf(mt, __shfl_xor(mt, 32, kWave)) * scale_log2;   // scale > 0: the max commutes
  float l_part = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], scale_log2, -mt));   // masked: 0
    sc[r] = p;
    l_part += p;
  }
  const float l = l_part + __shfl_xor(l_part, 32, kWave);
  floatx16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // the k slots of lane half h are keys {4h..4h+3, 8+4h..8+4h+3} of a 16-key
  // step for both operands: the lane's own probabilities r = 8kk..8kk+7
  const int n_kk = len > 16 ? 2 : 1;                         // keys 16..31 all masked otherwise
  for (int kk = 0; kk < n_kk; ++kk) {
    u32x4 pb;
#pragma unroll
    for (int e = 0; e < 4; ++e) pb[e] = pack_f16x2(sc[8 * kk + 2 * e], sc[8 * kk + 2 * e + 1]);
    const int kb = 16 * kk + 4 * half;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint32_t* vrow = reinterpret_cast<const uint32_t*>(&s_vt[32 * db + r32][0]) + kb / 2;   // 4-byte aligned
      o[db] = mfma32x16_f16(u32x4{vrow[0], vrow[1], vrow[4], vrow[5]}, pb, o[db]);
    }
  }
  if (r32 >= len) return;
  const float inv_l = 1.0f / l;                              // key 0 is always visible: l >= 1
  const size_t orow = (size_t(t0 + r32) * Hq + hq) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * db + 8 * rg + 4 * half;
      const float y0 = o[db][4 * rg] * inv_l, y1 = o[db][4 * rg + 1] * inv_l;
      const float y2 = o[db][4 * rg + 2] * inv_l, y3 = o[db][4 * rg + 3] * inv_l;
      if (out_fp8) {
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + orow + d0) =
            f2e4m3(y0 * out_inv) | (f2e4m3(y1 * out_inv) << 8) | (f2e4m3(y2 * out_inv) << 16) |
            (f2e4m3(y3 * out_inv) << 24);
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow + d0) =
            u32x2{pack_f16x2(y0, y1), pack_f16x2(y2, y3)};
      }
    }
}

void launch_rope_attn_small(const void* qkv, int n_seq, int max_len, int Hq, int Hkv, int d, float theta, float eps,
                            const int32_t* cu, const int32_t* cache_slot, const int32_t* used_keys, bool causal,
                            const void* qw, const void* kw, void* kc, void* vc, int capacity, void* out, bool fp8,
                            float out_inv, hipStream_t st, const float* tab) {
  (void)max_len;
  const RopeFreq freq = rope_freq(d, theta);
  const float scale_log2 = 1.4426950408889634f / __builtin_sqrtf(float(d));
  const dim3 grid(Hq, n_seq);
  auto go = [&](auto kern) {
    kern<<<grid, 64 * kSmallWaves, 0, st>>>(
        static_cast<const float*>(qkv), cu, cache_slot, used_keys, Hq, Hkv, causal ? 1 : 0, eps,
        static_cast<const uint16_t*>(qw), static_cast<const uint16_t*>(kw), static_cast<uint16_t*>(kc),
        static_cast<uint16_t*>(vc), capacity, scale_log2, out, fp8 ? 1 : 0, out_inv, tab, freq);
  };
  if (d == 128) go(rope_attn_small_kernel<128>);
  else go(rope_attn_small_kernel<64>);
}

}  // namespace hr
