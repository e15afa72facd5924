// GQA attention over the KV cache (step A4).
// Sources: flashrt-structures prefill_tower/fp8_chain.py, module docstring and
// `_prefill_mask_facts` (non-causal attention over exactly the used keys; pads
// trail, so a used-key count carries the mask) and `run` (attention between the
// cache write and the output projection); causal prefill for the bf16 chain of
// "Stabilize Higgs Audio termination and prefill", Summary.
//
// o_h[i] = sum_j softmax_j(q_h[i] . K_g[j] / sqrt(d)) V_g[j], g = h / (Hq/Hkv),
// j over [0, start_pos + i] (causal) or [0, used_keys) (non-causal).
//
// Workgroup = (query block, kv head g, sequence), 4 wavefronts.  The wavefronts
// share every K/V tile: they are the GROUP query heads of g (times 4/GROUP
// blocks of 16 positions).  Per 32-key tile:
//   S^T = K . Q^T   (A = 16 keys x 32 d from LDS, B = the wave's 16 queries,
//                    kept in registers) -> lane l holds query l%16 and keys
//                    4(l/16)+r of each 16-key half;
//   online softmax in base 2 per query (max over the 4 lanes of a column);
//   O^T += V^T . P^T (A = V^T from an LDS copy stored transposed, B = the
//                    lane's own 8 probabilities as bf16: the MFMA's k slots of
//                    lane group q are keys {4q..4q+3, 16+4q..16+4q+3} for both
//                    operands, so P needs no lane exchange).
// Probabilities feed the MFMA in bf16; sums and rescaling stay fp32.
#include "common.h"
#include "launch.h"

namespace hr {

constexpr int KT = 32;        // keys per tile
constexpr int VT_LD = 36;     // padded key stride of the transposed V tile (elements)

template <int DH, int GROUP>
__global__ __launch_bounds__(256) void attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ cache_slot, const int32_t* __restrict__ used_keys, int Hq, int Hkv,
    int capacity, int causal, float scale_log2, void* __restrict__ out, int out_fp8, float out_inv) {
  constexpr int QSUB = 4 / GROUP;             // 16-query sub-blocks per workgroup
  constexpr int QPW = 16 * QSUB;
  constexpr int K_LD = DH + 8;                // padded row of the K tile (elements)
  constexpr int NDS = DH / 32;                // 32-wide d steps of the score MFMA
  constexpr int NDB = DH / 16;                // 16-wide d blocks of the output
  __shared__ __attribute__((aligned(16))) uint16_t sK[KT * K_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[DH * VT_LD];

  const int s = blockIdx.z, g = blockIdx.y;
  const int len = cu[s + 1] - cu[s];
  const int qb = gridDim.x - 1 - blockIdx.x;  // longest causal rows first
  const int i0 = qb * QPW;
  if (i0 >= len) return;
  const int tok0 = cu[s];
  const int start = start_pos[s];
  const size_t base = size_t(cache_slot[s]) * capacity;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hg = wave % GROUP, qsub = wave / GROUP;
  const int h = g * GROUP + hg;
  const int lg = lane >> 4, rc = lane & 15;
  const int iq = i0 + qsub * 16 + rc;         // this lane's query (sequence-relative)
  const bool qok = iq < len;
  const int pos_q = start + iq;
  const int i_last = min(i0 + QPW, len) - 1;
  const int n_keys = causal ? start + i_last + 1 : used_keys[s];

  // the wave's queries as the B operand: query rc, d = 32 ds + 8 lg + [0,8)
  u32x4 qf[NDS];
  {
    const uint16_t* qrow = q + (size_t(tok0 + (qok ? iq : 0)) * Hq + h) * DH;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + ds * 32 + lg * 8);
      qf[ds] = qok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  floatx4 o[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) o[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_part = 0.f;

  const int n_tiles = (n_keys + KT - 1) / KT;
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int k0 = kt * KT;
    // K tile: 32 keys x DH -> sK[key][d]
    for (int c = tid; c < KT * (DH / 8); c += 256) {
      const int key = c / (DH / 8), d8 = c % (DH / 8);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k0 + key < n_keys)
        v = *reinterpret_cast<const u32x4*>(kc + ((base + k0 + key) * Hkv + g) * DH + d8 * 8);
      *reinterpret_cast<u32x4*>(sK + key * K_LD + d8 * 8) = v;
    }
    // V tile, transposed: sVt[d][key] as bf16 pairs of adjacent keys
    for (int c = tid; c < (KT / 2) * (DH / 8); c += 256) {
      const int kp = c % (KT / 2), d8 = c / (KT / 2);
      const int key = 2 * kp;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (k0 + key < n_keys)
        a = *reinterpret_cast<const u32x4*>(vc + ((base + k0 + key) * Hkv + g) * DH + d8 * 8);
      if (k0 + key + 1 < n_keys)
        b = *reinterpret_cast<const u32x4*>(vc + ((base + k0 + key + 1) * Hkv + g) * DH + d8 * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (a[j] & 0xFFFFu) | (b[j] << 16);
        const uint32_t hi = (a[j] >> 16) | (b[j] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(sVt + (d8 * 8 + 2 * j) * VT_LD + key) = lo;
        *reinterpret_cast<uint32_t*>(sVt + (d8 * 8 + 2 * j + 1) * VT_LD + key) = hi;
      }
    }
    __syncthreads();

    // scores for keys 16 hb + 4 lg + r, query rc
    floatx4 sc[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        u32x4 kf = *reinterpret_cast<const u32x4*>(sK + (hb * 16 + rc) * K_LD + ds * 32 + lg * 8);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf),
                                                    __builtin_bit_cast(bf16x8, qf[ds]), a, 0, 0, 0);
      }
      sc[hb] = a;
    }
    float mt = -__builtin_inff();
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = k0 + hb * 16 + lg * 4 + r;
        const bool vis = j < n_keys && (!causal || j <= pos_q);
        const float v = vis ? sc[hb][r] * scale_log2 : -__builtin_inff();
        sc[hb][r] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[hb][r] = exp2f(sc[hb][r] - m_use);
        psum += p[hb][r];
      }
    l_part = l_part * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < NDB; ++j) o[j] *= alpha;
    u32x4 pb;
    pb[0] = pack_bf2(p[0][0], p[0][1]);
    pb[1] = pack_bf2(p[0][2], p[0][3]);
    pb[2] = pack_bf2(p[1][0], p[1][1]);
    pb[3] = pack_bf2(p[1][2], p[1][3]);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t* vrow = sVt + (db * 16 + rc) * VT_LD;
      u32x2 x0 = *reinterpret_cast<const u32x2*>(vrow + 4 * lg);
      u32x2 x1 = *reinterpret_cast<const u32x2*>(vrow + 16 + 4 * lg);
      u32x4 va = {x0[0], x0[1], x1[0], x1[1]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                      __builtin_bit_cast(bf16x8, pb), o[db], 0, 0, 0);
    }
    __syncthreads();
  }

  float l = l_part;
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  const float inv_l = l > 0.f ? 1.0f / l : 0.f;
  if (!qok) return;
  const size_t orow = (size_t(tok0 + iq) * Hq + h) * DH;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d0 = db * 16 + 4 * lg;
    float y0 = o[db][0] * inv_l, y1 = o[db][1] * inv_l, y2 = o[db][2] * inv_l, y3 = o[db][3] * inv_l;
    if (out_fp8) {
      uint32_t w = f2e4m3(y0 * out_inv) | (f2e4m3(y1 * out_inv) << 8) | (f2e4m3(y2 * out_inv) << 16) |
                   (f2e4m3(y3 * out_inv) << 24);
      *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + orow + d0) = w;
    } else {
      u32x2 w = {pack_bf2(y0, y1), pack_bf2(y2, y3)};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow + d0) = w;
    }
  }
}

template <int DH, int GROUP>
static void launch_attn_t(const void* q, const void* kc, const void* vc, const int32_t* cu,
                          const int32_t* sp, const int32_t* slot, const int32_t* used, int n_seq,
                          int max_len, int Hq, int Hkv, int cap, bool causal, void* out, bool fp8,
                          float out_inv, hipStream_t st) {
  constexpr int QPW = 16 * (4 / GROUP);
  dim3 grid((max_len + QPW - 1) / QPW, Hkv, n_seq);
  const float scale_log2 = 1.4426950408889634f / __builtin_sqrtf(float(DH));
  attention_kernel<DH, GROUP><<<grid, 256, 0, st>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
      static_cast<const uint16_t*>(vc), cu, sp, slot, used, Hq, Hkv, cap, causal ? 1 : 0,
      scale_log2, out, fp8 ? 1 : 0, out_inv);
}

void launch_attention(const void* q, const void* kc, const void* vc, const int32_t* cu,
                      const int32_t* sp, const int32_t* slot, const int32_t* used, int n_seq,
                      int max_len, int Hq, int Hkv, int d, int cap, bool causal, void* out, bool fp8,
                      float out_inv, hipStream_t st) {
  const int group = Hq / Hkv;
#define HR_ATT(DH_, G_)                                                                         \
  if (d == DH_ && group == G_) {                                                                \
    launch_attn_t<DH_, G_>(q, kc, vc, cu, sp, slot, used, n_seq, max_len, Hq, Hkv, cap, causal, \
                           out, fp8, out_inv, st);                                              \
    return;                                                                                     \
  }
  HR_ATT(128, 4) HR_ATT(128, 2) HR_ATT(128, 1) HR_ATT(64, 4) HR_ATT(64, 2) HR_ATT(64, 1)
#undef HR_ATT
}

}  // namespace hr
