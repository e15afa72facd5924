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
// Workgroup = (query block, kv head g, sequence), 4 wavefronts sharing every
// K/V tile: the GROUP query heads of g, times 4/GROUP blocks of 32 positions.
// Per 64-key tile, with v_mfma_f32_32x32x16_f16 (q in fp16; the bf16 K and V
// rows convert exactly to fp16 as they are staged in LDS):
//   S^T = K . Q^T  (A = 32 keys x 16 d from LDS, B = the wave's 32 queries,
//                   kept in registers) -> lane l holds query l%32 and keys
//                   8(r/4) + 4(l/32) + r%4, r = 0..15, of each 32-key block;
//   online softmax in base 2 per query (the other half of a query's keys is in
//                   lane l^32: one exchange);
//   O^T += V^T . P^T: the MFMA's 8 k slots of lane half h are keys
//                   {4h..4h+3, 8+4h..8+4h+3} of a 16-key step for BOTH operands,
//                   which are exactly the lane's own probabilities r = 8kk..8kk+7,
//                   so P goes from the score accumulator to the B operand with no
//                   lane exchange; V is staged transposed in LDS.
// The next tile's K and V are fetched into registers while the current tile is
// computed.  Probabilities feed the MFMA in fp16; sums and rescaling stay fp32.
#include "common.h"
#include "launch.h"
#include "rope_math.h"

namespace hr {

constexpr int AKT = 64;        // keys per tile
constexpr int VT_LD = 72;      // padded key stride of the transposed V tile (elements)

__device__ __forceinline__ floatx16 mfma32_f16(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// wait until at most N of this thread's vector-memory loads are outstanding
template <int N>
__device__ __forceinline__ void wait_vm_f16() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// workgroup barrier without waiting for this thread's memory operations (the
// copies it publishes were waited for); the empty asm keeps LDS accesses on
// their side of it
__device__ __forceinline__ void lds_barrier_f16() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Key chunks of a query block with n_tiles 64-key tiles: at least chunk_tiles
// tiles per chunk, and no more chunks than n_slots (longer rows take longer
// chunks).  chunk_tiles == 0: one chunk.
__device__ __forceinline__ void chunk_plan(int n_tiles, int chunk_tiles, int n_slots, int& ct, int& n_chunks) {
  if (chunk_tiles <= 0 || n_tiles <= chunk_tiles) {
    ct = n_tiles;
    n_chunks = 1;
    return;
  }
  ct = max(chunk_tiles, (n_tiles + n_slots - 1) / n_slots);
  n_chunks = (n_tiles + ct - 1) / ct;
}

// NG groups of wavefronts: group n takes key tiles kt0 + n, kt0 + n + NG, ...
// of the same queries, with its own K/V buffers; the groups' running
// (max, sum, output) are merged through LDS at the end.  NG = 2 gives a long
// row two wavefronts per SIMD that hide each other's latencies.  HSPLIT = 2
// gives each of two workgroups half the GROUP query heads of a KV head (each
// stages the same K/V tiles): twice the workgroups, half the work per CU for
// grids that would leave CUs idle.
template <int DH, int GROUP, int NG, int HSPLIT = 1>
__global__ __launch_bounds__(64 * (GROUP / HSPLIT) * (4 / GROUP) * NG) __attribute__((amdgpu_waves_per_eu(2)))
void attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ cache_slot, const int32_t* __restrict__ used_keys, int Hq, int Hkv,
    int capacity, int causal, float scale_log2, void* __restrict__ out, int out_fp8, float out_inv,
    int chunk_tiles, int n_slots, float* __restrict__ part_o, float2_t* __restrict__ part_ml, int T) {
  constexpr int QSUB = 4 / GROUP;             // 32-query sub-blocks per workgroup
  constexpr int QPW = 32 * QSUB;
  constexpr int HPW = GROUP / HSPLIT;         // query heads per workgroup
  constexpr int GT = 64 * HPW * QSUB;         // threads of one key-tile group
  static_assert(GROUP % HSPLIT == 0, "heads split evenly");
  constexpr int K_LD = DH + 8;                // padded row of the K tile (elements)
  constexpr int NKS = DH / 16;                // 16-wide d steps of the score MFMA
  constexpr int NDB = DH / 32;                // 32-wide d blocks of the output
  constexpr int KCH = AKT * (DH / 8);         // 16-byte chunks of a K (or V) tile
  constexpr int KPT = KCH / GT;               // K chunks per thread
  constexpr int VPT = KCH / 2 / GT;           // V key-pair units per thread (2 loads each)
  static_assert(KPT >= 1 && VPT >= 1, "tile / thread mapping");
  constexpr int kGroupLds = AKT * K_LD + DH * VT_LD;   // elements of one group's K and V^T tiles
  __shared__ __attribute__((aligned(16))) uint16_t smem[NG * kGroupLds];

  const int s = blockIdx.z, g = int(blockIdx.y) / HSPLIT, hsel = int(blockIdx.y) % HSPLIT;
  const int len = cu[s + 1] - cu[s];
  // blockIdx.x = (query block, key chunk slot); longest causal rows first
  const int qb = gridDim.x / n_slots - 1 - int(blockIdx.x) / n_slots;
  const int ck = int(blockIdx.x) % n_slots;
  const int i0 = qb * QPW;
  if (i0 >= len) return;
  const int tok0 = cu[s];
  const int start = start_pos[s];
  const size_t base = size_t(cache_slot[s]) * capacity;
  const int lane = threadIdx.x & 63;
  const int grp = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / GT);   // key-tile group (wave-uniform)
  const int tid = int(threadIdx.x) % GT, wave = tid >> 6;   // within the group
  uint16_t* sK = smem + grp * kGroupLds;
  uint16_t* sVt = sK + AKT * K_LD;
  const int hg = wave % HPW, qsub = wave / HPW;
  const int hh = g * GROUP + hsel * HPW + hg;
  const int half = lane >> 5, r32 = lane & 31;
  const int iq = i0 + qsub * 32 + r32;        // this lane's query (sequence-relative)
  const bool qok = iq < len;
  const int pos_q = start + iq;
  const int i_last = min(i0 + QPW, len) - 1;
  const int n_keys = causal ? start + i_last + 1 : used_keys[s];
  // key chunk: tiles [kt0, kt1) of this query block (all of them when not split)
  const int n_tiles_all = (n_keys + AKT - 1) / AKT;
  int ct, n_chunks;
  chunk_plan(n_tiles_all, chunk_tiles, n_slots, ct, n_chunks);
  if (ck >= n_chunks) return;
  const bool split = n_chunks > 1;
  const int kt0 = ck * ct;
  const int kt1 = min(n_tiles_all, kt0 + ct);

  // the wave's queries as the B operand: query r32, d = 16 ks + 8 half + [0,8).
  // A lane past the block's end takes the sequence's first query instead (its
  // finite results are never stored); no select on the loaded values, so the
  // first K/V fetch below issues while these loads are in flight.
  u32x4 qf[NKS];
  {
    const uint16_t* qrow = q + (size_t(tok0 + (qok ? iq : 0)) * Hq + hh) * DH;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + half * 8);
  }

  // K/V tile fetch into registers: K chunk c -> (key c / (DH/8), d8 c % (DH/8));
  // V unit u -> key pair (u % 32) of the tile, d8 = u / 32.  Keys past the end
  // read the last key's row instead (a written, finite row): their scores are
  // masked to -inf, so they add 0 x finite.
  u32x4 rk[KPT], rv[VPT][2];
  const uint16_t* kbase = kc + (base * Hkv + g) * DH;
  const uint16_t* vbase = vc + (base * Hkv + g) * DH;
  const size_t row_stride = size_t(Hkv) * DH;
  const int last_key = n_keys - 1;
  // A thread's chunk j is its chunk 0 moved by a uniform step: KROWS rows
  // for K, VCOLS elements for V.  So a tile inside the keys is fetched from a
  // uniform base plus one byte offset per thread (scalar base + vector offset
  // addressing: no per-load address arithmetic).
  static_assert(GT % (DH / 8) == 0 && GT % (AKT / 2) == 0, "uniform chunk steps");
  constexpr int KROWS = GT / (DH / 8);
  constexpr int VCOLS = GT / (AKT / 2) * 8;
  const uint32_t k_off = (uint32_t(tid / (DH / 8)) * uint32_t(row_stride) + uint32_t(tid % (DH / 8)) * 8) * 2;
  const uint32_t v_off = (uint32_t(2 * (tid % (AKT / 2))) * uint32_t(row_stride) + uint32_t(tid / (AKT / 2)) * 8) * 2;
  auto fetch = [&](int k0) {
    if (k0 + AKT <= n_keys) {          // uniform: no row of the tile past the keys
      const uint8_t* kt = reinterpret_cast<const uint8_t*>(kbase + size_t(k0) * row_stride);
      const uint8_t* vt = reinterpret_cast<const uint8_t*>(vbase + size_t(k0) * row_stride);
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        rk[j] = *reinterpret_cast<const u32x4*>(kt + size_t(j) * KROWS * row_stride * 2 + k_off);
#pragma unroll
      for (int j = 0; j < VPT; ++j)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          rv[j][e] = *reinterpret_cast<const u32x4*>(vt + (size_t(e) * row_stride + j * VCOLS) * 2 + v_off);
      return;
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int c = tid + GT * j;
      const int key = c / (DH / 8), d8 = c % (DH / 8);
      const int row = min(k0 + key, last_key);
      rk[j] = *reinterpret_cast<const u32x4*>(kbase + size_t(row) * row_stride + d8 * 8);
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int u = tid + GT * j;
      const int key = 2 * (u % (AKT / 2)), d8 = u / (AKT / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = min(k0 + key + e, last_key);
        rv[j][e] = *reinterpret_cast<const u32x4*>(vbase + size_t(row) * row_stride + d8 * 8);
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int c = tid + GT * j;
      const int key = c / (DH / 8), d8 = c % (DH / 8);
      *reinterpret_cast<u32x4*>(sK + key * K_LD + d8 * 8) = bf8_to_f16x8(rk[j]);
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int u = tid + GT * j;
      const int key = 2 * (u % (AKT / 2)), d8 = u / (AKT / 2);
      const u32x4 a = bf8_to_f16x8(rv[j][0]), b = bf8_to_f16x8(rv[j][1]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *reinterpret_cast<uint32_t*>(sVt + (d8 * 8 + 2 * w) * VT_LD + key) = (a[w] & 0xFFFFu) | (b[w] << 16);
        *reinterpret_cast<uint32_t*>(sVt + (d8 * 8 + 2 * w + 1) * VT_LD + key) =
            (a[w] >> 16) | (b[w] & 0xFFFF0000u);
      }
    }
  };

  floatx16 o[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
  float m_run = -__builtin_inff();
  float l_part = 0.f;

  if (kt0 + grp < kt1) fetch((kt0 + grp) * AKT);
  // q and the first tile land before the loop (the first staging needs the
  // tile anyway).  Without this explicit wait the compiler, seeing the q loads
  // possibly in flight at the loop head, guards the score MFMAs of every tile
  // with waits that also cover the next tile's prefetch (vmcnt(7) .. vmcnt(0)
  // right after the prefetch issues), serialising each fetch with the math.
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));   // vmcnt(0) only
  for (int kb = kt0; kb < kt1; kb += NG) {
    const int kt = kb + grp;
    const bool have = kt < kt1;      // the other group may still have a tile
    const int k0 = kt * AKT;
    __syncthreads();                 // every wave is done with the previous tile
    if (have) stage();
    __syncthreads();
    if (kt + NG < kt1) fetch(k0 + NG * AKT);   // in flight during this tile's math
    if (!have) continue;

    // scores of 2 blocks of 32 keys
    floatx16 sc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      floatx16 a;
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(sK + (blk * 32 + r32) * K_LD + ks * 16 + half * 8);
        a = mfma32_f16(kf, qf[ks], a);
      }
      sc[blk] = a;
    }
    // masks only where the tile crosses the causal diagonal of this wave's
    // queries or the end of the keys (wave-uniform test)
    const int wave_pos0 = start + i0 + qsub * 32;
    const bool need_mask = (k0 + AKT > n_keys) || (causal && k0 + AKT - 1 > wave_pos0);
    if (need_mask) {
      // causal: key j visible to query pos_q iff j <= pos_q (which is < n_keys)
      const int j_max = causal ? pos_q : last_key;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + blk * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (j > j_max) sc[blk][r] = -__builtin_inff();
        }
    }
    float mt = -__builtin_inff();
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[blk][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave)) * scale_log2;   // scale > 0: max commutes
    // The reference max m_run moves only when a tile exceeds it by more than
    // 8 (base 2): probabilities then stay <= 2^8, well inside fp16 and fp32
    // range at unchanged relative precision, and most tiles skip rescaling
    // the accumulators (the result o / l does not depend on the reference).
    const bool grow = mt > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;   // 0 from -inf
      if (grow) m_run = mt;
      l_part *= alpha;
#pragma unroll
      for (int j = 0; j < NDB; ++j) o[j] *= alpha;
    }
    const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[blk][r], scale_log2, -m_use));
        sc[blk][r] = p;
        psum += p;
      }
    l_part += psum;
    // O^T += V^T P^T, 4 MFMAs (2 blocks x 2 k-steps of 16 keys) per d block
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pb;
        pb[0] = pack_f16x2(sc[blk][8 * kk + 0], sc[blk][8 * kk + 1]);
        pb[1] = pack_f16x2(sc[blk][8 * kk + 2], sc[blk][8 * kk + 3]);
        pb[2] = pack_f16x2(sc[blk][8 * kk + 4], sc[blk][8 * kk + 5]);
        pb[3] = pack_f16x2(sc[blk][8 * kk + 6], sc[blk][8 * kk + 7]);
        const int kb = blk * 32 + kk * 16 + 4 * half;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* vrow = sVt + (db * 32 + r32) * VT_LD;
          const u32x2 x0 = *reinterpret_cast<const u32x2*>(vrow + kb);
          const u32x2 x1 = *reinterpret_cast<const u32x2*>(vrow + kb + 8);
          const u32x4 va = {x0[0], x0[1], x1[0], x1[1]};
          o[db] = mfma32_f16(va, pb, o[db]);
        }
      }
  }

  if constexpr (NG > 1) {
    // merge the groups' partial softmaxes into group 0 (through the now idle
    // tile buffers: GT lanes x (2 + 16 NDB) floats per group)
    constexpr int kVals = 2 + 16 * NDB;
    static_assert(size_t(NG - 1) * GT * kVals * 4 <= sizeof(smem), "merge buffer");
    float* xch = reinterpret_cast<float*>(smem);
    __syncthreads();
    if (grp > 0) {
      float* my = xch + (size_t(grp - 1) * GT + tid) * kVals;
      my[0] = m_run;
      my[1] = l_part;
#pragma unroll
      for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) my[2 + 16 * j + r] = o[j][r];
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g2 = 1; g2 < NG; ++g2) {
      const float* ot = xch + (size_t(g2 - 1) * GT + tid) * kVals;
      const float m2 = ot[0];
      const float mm = fmaxf(m_run, m2);
      const float a1 = (m_run == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
      const float a2 = (m2 == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m2 - mm);
      l_part = l_part * a1 + ot[1] * a2;
#pragma unroll
      for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] = o[j][r] * a1 + ot[2 + 16 * j + r] * a2;
      m_run = mm;
    }
  }
  float l = l_part + __shfl_xor(l_part, 32, kWave);
  if (!qok) return;
  if (split) {
    // partial of this key chunk: unnormalised o, running max (log2 units), sum
    const size_t prow = (size_t(ck) * T + tok0 + iq) * Hq + hh;
    float* po = part_o + prow * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = db * 32 + 8 * rg + 4 * half;
        *reinterpret_cast<floatx4*>(po + d0) =
            floatx4{o[db][4 * rg], o[db][4 * rg + 1], o[db][4 * rg + 2], o[db][4 * rg + 3]};
      }
    if (half == 0) part_ml[prow] = float2_t{m_run, l};
    return;
  }
  const float inv_l = l > 0.f ? 1.0f / l : 0.f;
  const size_t orow = (size_t(tok0 + iq) * Hq + hh) * DH;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = db * 32 + 8 * rg + 4 * half;
      const float y0 = o[db][4 * rg] * inv_l, y1 = o[db][4 * rg + 1] * inv_l;
      const float y2 = o[db][4 * rg + 2] * inv_l, y3 = o[db][4 * rg + 3] * inv_l;
      if (out_fp8) {
        const uint32_t w = f2e4m3(y0 * out_inv) | (f2e4m3(y1 * out_inv) << 8) |
                           (f2e4m3(y2 * out_inv) << 16) | (f2e4m3(y3 * out_inv) << 24);
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + orow + d0) = w;
      } else {
        const u32x2 w = {pack_f16x2(y0, y1), pack_f16x2(y2, y3)};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow + d0) = w;
      }
    }
}

// Combine the key-chunk partials of the split query blocks:
// o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c, M = max_c m_c, taken as
// one pass with a running maximum.  Grid (token, 256 (head, 4-dim) units per
// workgroup); rows of unsplit query blocks were written final.
template <int DH>
__global__ __launch_bounds__(256) void attention_merge_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ start_pos, const int32_t* __restrict__ used_keys,
    int n_seq, int Hq, int causal, int qpw, int chunk_tiles, int n_slots, const float* __restrict__ part_o,
    const float2_t* __restrict__ part_ml, int T, void* __restrict__ out, int out_fp8, float out_inv) {
  const int t = blockIdx.x;
  const int s = find_seq(cu, n_seq, t);
  const int i = t - cu[s], len = cu[s + 1] - cu[s];
  const int i_last = min((i / qpw) * qpw + qpw, len) - 1;
  const int n_keys = causal ? start_pos[s] + i_last + 1 : used_keys[s];
  int ct, nch;
  chunk_plan((n_keys + AKT - 1) / AKT, chunk_tiles, n_slots, ct, nch);
  if (nch <= 1) return;
  // thread: one head and 4 output dims; one pass over the chunks with a
  // running maximum (unrolled, so the chunks' loads are in flight together)
  const int u = blockIdx.y * 256 + threadIdx.x;
  if (u >= Hq * (DH / 4)) return;
  const int h = u / (DH / 4), d4 = u % (DH / 4);
  float M = -__builtin_inff(), L = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int c = 0; c < nch; ++c) {
    const size_t prow = (size_t(c) * T + t) * Hq + h;
    const float2_t ml = part_ml[prow];
    const floatx4 o = *reinterpret_cast<const floatx4*>(part_o + prow * DH + 4 * d4);
    const float mn = fmaxf(M, ml[0]);
    const float a = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - mn);
    const float b = ml[0] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ml[0] - mn);
    L = L * a + b * ml[1];
    acc = acc * a + b * o;
    M = mn;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const size_t orow = (size_t(t) * Hq + h) * DH + 4 * d4;
  const float y0 = acc[0] * inv, y1 = acc[1] * inv, y2 = acc[2] * inv, y3 = acc[3] * inv;
  if (out_fp8) {
    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + orow) =
        f2e4m3(y0 * out_inv) | (f2e4m3(y1 * out_inv) << 8) | (f2e4m3(y2 * out_inv) << 16) |
        (f2e4m3(y3 * out_inv) << 24);
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow) = u32x2{pack_f16x2(y0, y1), pack_f16x2(y2, y3)};
  }
}

// ============================================================ attention over fp16 copies
// A batch whose keys are all its own rows (every sequence from position 0)
// and whose QKV launch also wrote fp16 copies of its K and V rows
// ([Tp][Hkv][d]): the tiles need no conversion, so they go HBM -> LDS by
// global_load_lds (no register round trip, no VALU).  A workgroup takes one
// query head and the query blocks p and nb-1-p of a sequence (32 rows each;
// causal: the longest and the shortest rows together, so every workgroup of a
// prompt has the same number of tiles), as 8 waves: 4 tile streams, stream j
// taking the 32-key tiles j, j+4, j+8, ... of the longer block, each stream
// with a wave for each block (the shorter block's wave computes the tiles its
// rows reach; both copy: the longer block's wave the k half, the other the v
// half).  One barrier per step of 4 tiles; each stream double-buffers its
// tiles (2 x 2 x 8 KB at d 128).  Workgroup ids are dealt with the kv head
// varying fastest, so all workgroups of one kv head share an XCD's L2.  Per
// tile and wave, as in attention_kernel: S^T = K Q^T with
// v_mfma_f32_32x32x16_f16 (lane: query l % 32, keys 8(r/4) + 4(l/32) + r%4),
// the online softmax in base 2 (reference max moved only when exceeded by
// more than 8), O^T += V^T P^T with the lane's own fp16 probabilities as the B
// operand; the V^T fragment (4 consecutive keys of one d per read) comes from
// the row-major V tile through ds_read_b64_tr_b16: in each group of 16 lanes,
// lane i = 4e + q supplies the address of 4 elements of row e, and lane
// 4q + c receives element c of rows 0..3 -- so lane i points at key K0 + i/4,
// dims 4(i%4)..+3 of its 16-dim group.  The copies are swizzled on the global
// side so the fragment reads hit distinct banks (k rows of 16 chunks: chunk c
// of row r at c ^ (r % 16), of 8: c ^ ((r / 2) % 8); v rows: c ^ 4 (r % 4),
// of 8 chunks c ^ 4 ((r / 2) % 2)).  At the end the 4 streams of a block merge
// their (max, sum, output) through LDS in stream order, and the normalised
// rows are staged in LDS so they leave as whole 16-byte row chunks.  Rows
// past the copies' last row read that row (finite; their scores are masked).
constexpr int kF16Streams = 4;               // tile streams of a workgroup
constexpr int kF16Waves = 2 * kF16Streams;   // a long-block and a short-block wave per stream
constexpr int kF16KT = 32;                   // keys per tile

template <int DH>
constexpr size_t attention_f16_lds() { return size_t(kF16Streams) * 2 * 2 * kF16KT * DH * 2; }

// max of a lane's value and lane l ^ 32's (v_permlane32_swap: one VALU, no LDS)
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_dma16(const void* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

template <int DH>
__global__ __launch_bounds__(64 * kF16Waves) void attention_f16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k16, const uint16_t* __restrict__ v16, int Tp,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ used_keys, int Hq, int Hkv, int causal,
    float scale_log2, void* __restrict__ out, int out_fp8, float out_inv) {
  constexpr int KT = kF16KT;
  constexpr int NKS = DH / 16, NDB = DH / 32;
  constexpr int KCH = DH / 8;                // 16-byte chunks of a row
  constexpr int TB = KT * DH * 2;            // bytes of a k tile (and of a v tile)
  constexpr int NCP = TB / 1024;             // 1-KB wave copies per tile half
  constexpr int STAGE = 2 * TB;
  static_assert(TB % 1024 == 0, "whole wave copies");
  extern __shared__ __attribute__((aligned(16))) uint8_t f16_smem[];

  // workgroup id -> (query-block pair, head) with the kv head varying
  // fastest: consecutive ids go to the 8 XCDs in turn, so every workgroup of
  // one kv head runs on one XCD and its K / V tiles are shared in that L2
  const int G = Hq / Hkv;
  const int wid = int(blockIdx.x) + int(gridDim.x) * int(blockIdx.y);
  const int g = wid % Hkv, rest = wid / Hkv;
  const int hh = g * G + rest % G, p = rest / G;
  const int s = blockIdx.z;
  const int tok0 = cu[s], len = cu[s + 1] - tok0;
  const int nb = (len + 31) / 32;
  const int b_long = nb - 1 - p;
  if (p > b_long) return;                    // whole workgroup, before any barrier
  const bool single = p == b_long;
  const int used = causal ? 0 : used_keys[s];
  const int nk_l = causal ? min(32 * b_long + 31, len - 1) + 1 : used;
  const int nk_s = single ? 0 : (causal ? 32 * p + 32 : used);
  const int t_l = (nk_l + KT - 1) / KT, t_s = (nk_s + KT - 1) / KT;
  const int n_steps = (t_l + kF16Streams - 1) / kF16Streams;   // t_l >= t_s
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int js = wave % kF16Streams;         // stream: tiles js, js + 4, js + 8, ...
  const bool is_short = wave >= kF16Streams;
  const int blk = is_short ? p : b_long;
  const int n_my = is_short ? t_s : t_l;     // tiles of this wave's block
  const int n_keys = is_short ? nk_s : nk_l;

  const int half = lane >> 5, r32 = lane & 31;
  const int i0 = 32 * blk;
  const int iq = i0 + r32;                   // this lane's query (sequence-relative)
  u32x4 qf[NKS];
  {
    const uint16_t* qrow = q + (size_t(tok0 + (iq < len ? iq : 0)) * Hq + hh) * DH;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + half * 8);
  }

  // the stream's tiles: the long-block wave copies the k half, the short-block
  // wave the v half (a thread's copy i of a tile is its copy i of tile 0 moved
  // by a uniform step of KT rows: a uniform base plus one byte offset)
  uint8_t* sl_base = f16_smem + size_t(js) * 2 * STAGE;
  const size_t krow = size_t(Hkv) * DH * 2;                    // bytes from one key row to the next
  const uint8_t* src = reinterpret_cast<const uint8_t*>(is_short ? v16 : k16) + (size_t(tok0) * Hkv + g) * DH * 2;
  const int key_last = Tp - tok0 - 1;                          // last row of the copies (relative)
  auto kswz_of = [](int r) { return KCH == 16 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz_of = [](int r) { return KCH == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  uint32_t off[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    const int sl = 64 * i + lane, r = sl / KCH;
    off[i] = uint32_t(r) * uint32_t(krow) + uint32_t((sl % KCH) ^ (is_short ? vswz_of(r) : kswz_of(r))) * 16;
  }
  auto fetch = [&](int t, int stg) {
    uint8_t* dst = sl_base + stg * STAGE + (is_short ? TB : 0);
    if (t * KT + KT - 1 <= key_last) {       // uniform: the whole tile inside the copies
      const uint8_t* base = src + size_t(t) * KT * krow;
#pragma unroll
      for (int i = 0; i < NCP; ++i) lds_dma16(base + off[i], dst + i * 1024);
      return;
    }
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int sl = 64 * i + lane, r = sl / KCH;
      lds_dma16(src + size_t(min(t * KT + r, key_last)) * krow + ((sl % KCH) ^ (is_short ? vswz_of(r) : kswz_of(r))) * 16,
                dst + i * 1024);
    }
  };

  floatx16 o[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
  float m_run = -__builtin_inff();
  float l_part = 0.f;
  const int kswz = kswz_of(r32);
  // the lane's transposed-read address in a v tile, relative to key 16 kk +
  // 8 x and dim block db: row 4 (lane / 32) + (lane % 16) / 4, dims
  // 16 ((lane / 16) % 2) + 4 (lane % 4) .. + 3 (a half chunk)
  const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  if (js < t_l) fetch(js, 0);
  for (int k = 0; k < n_steps; ++k) {
    wait_vm_f16<0>();                        // this wave's half of step k (and q) landed
    lds_barrier_f16();                       // both halves landed; step k-1's stage is free
    const int t = k * kF16Streams + js;
    if (t + kF16Streams < t_l) fetch(t + kF16Streams, (k + 1) & 1);
    if (t >= n_my) continue;
    const uint8_t* sk = sl_base + (k & 1) * STAGE;
    const uint8_t* sv = sk + TB;
    const int k0 = t * KT;
    // the k fragments ahead of the score MFMAs, then the v fragments, whose
    // reads overlap the softmax (registers: the v reads reuse the k ones)
    u32x4 kf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kf[ks] = *reinterpret_cast<const u32x4*>(sk + (r32 * KCH + ((2 * ks + half) ^ kswz)) * 16);
    __builtin_amdgcn_sched_barrier(0);
    floatx16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sc = mfma32_f16(kf[ks], qf[ks], sc);
    u32x2 vf[2][NDB][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int r = 16 * kk + 8 * x + tr_row, vs = vswz_of(r);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int dd = 32 * db + tr_dim;
          const uint8_t* a = sv + r * (DH * 2) + (((dd >> 3) ^ vs) << 4) + (dd & 7) * 2;
          vf[kk][db][x] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(a)));
        }
      }
    __builtin_amdgcn_sched_barrier(0);
    const bool need_mask = causal ? (k0 + KT - 1 > i0) : (k0 + KT > n_keys);
    if (need_mask) {
      const int j_max = causal ? iq : n_keys - 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (j > j_max) sc[r] = -__builtin_inff();
      }
    }
    float mt = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = max_xor32(mt) * scale_log2;         // scale > 0: max commutes
    const bool grow = mt > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;   // 0 from -inf
      if (grow) m_run = mt;
      l_part *= alpha;
#pragma unroll
      for (int j = 0; j < NDB; ++j) o[j] *= alpha;
    }
    const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], scale_log2, -m_use));
      sc[r] = pr;
      psum += pr;
    }
    l_part += psum;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[e] = pack_f16x2(sc[8 * kk + 2 * e], sc[8 * kk + 2 * e + 1]);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        o[db] = mfma32_f16(u32x4{vf[kk][db][0][0], vf[kk][db][0][1], vf[kk][db][1][0], vf[kk][db][1][1]}, pb, o[db]);
    }
  }

  // merge each block's streams (fixed order) through the now idle LDS: the
  // stream-0 wave of a block keeps its state, the other three post theirs
  // (value-major, so a wave's 64 lanes write 256 contiguous bytes)
  constexpr int kVals = 2 + 16 * NDB;
  constexpr size_t kMerge = size_t(2 * (kF16Streams - 1)) * kVals * 64 * 4;
  constexpr int SROW = DH * 2 + 16;          // a staged output row (bytes; 16 apart in banks)
  static_assert(kMerge + 2 * 32 * SROW <= attention_f16_lds<DH>(), "merge and staging buffers");
  float* xch = reinterpret_cast<float*>(f16_smem);
  __syncthreads();                           // every wave is done with its tiles
  const int slot0 = (is_short ? 1 : 0) * (kF16Streams - 1);
  if (js > 0) {
    float* my = xch + size_t(slot0 + js - 1) * kVals * 64 + lane;
    my[0] = m_run;
    my[64] = l_part;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) my[(2 + 16 * j + r) * 64] = o[j][r];
  }
  __syncthreads();
  if (js > 0 || (is_short && single)) return;
#pragma unroll 1
  for (int w2 = 1; w2 < kF16Streams; ++w2) {
    const float* ot = xch + size_t(slot0 + w2 - 1) * kVals * 64 + lane;
    const float m2 = ot[0];
    const float mm = fmaxf(m_run, m2);
    const float a1 = (m_run == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
    const float a2 = (m2 == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m2 - mm);
    l_part = l_part * a1 + ot[64] * a2;
#pragma unroll
    for (int j = 0; j < NDB; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[j][r] = o[j][r] * a1 + ot[(2 + 16 * j + r) * 64] * a2;
      __builtin_amdgcn_sched_barrier(0);     // 16 values in flight at a time (registers)
    }
    m_run = mm;
  }
  const float l = l_part + __shfl_xor(l_part, 32, kWave);
  const float inv_l = l > 0.f ? 1.0f / l : 0.f;
  // the block's normalised rows go to LDS (this wave's own staging area) and
  // leave as whole 16-byte chunks of a row: a lane's accumulators hold 4
  // dims of one query, so direct stores would write 8 bytes per row and lane
  uint8_t* stg = f16_smem + kMerge + (is_short ? 32 * SROW : 0);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = db * 32 + 8 * rg + 4 * half;
      const float y0 = o[db][4 * rg] * inv_l, y1 = o[db][4 * rg + 1] * inv_l;
      const float y2 = o[db][4 * rg + 2] * inv_l, y3 = o[db][4 * rg + 3] * inv_l;
      if (out_fp8)
        *reinterpret_cast<uint32_t*>(stg + r32 * SROW + d0) =
            f2e4m3(y0 * out_inv) | (f2e4m3(y1 * out_inv) << 8) | (f2e4m3(y2 * out_inv) << 16) |
            (f2e4m3(y3 * out_inv) << 24);
      else
        *reinterpret_cast<u32x2*>(stg + r32 * SROW + 2 * d0) = u32x2{pack_f16x2(y0, y1), pack_f16x2(y2, y3)};
    }
  const int eb = out_fp8 ? 1 : 2;            // output bytes per element
  const int cpr = DH * eb / 16;              // 16-byte chunks per row
  const int rpi = kWave / cpr;               // rows per store instruction
  for (int r0 = 0; r0 < 32; r0 += rpi) {
    const int r = r0 + lane / cpr, c = lane % cpr;
    if (i0 + r < len) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * SROW + c * 16);
      *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(out) + (size_t(tok0 + i0 + r) * Hq + hh) * DH * eb + c * 16) = v;
    }
  }
}

// ============================================================ decode attention
// One query row per sequence (a decode step).  Workgroup = (key chunk, kv
// head, sequence), 4 waves.  The chunk's keys are dealt KPW to a wave
// instruction, DH/8 lanes per key (lane: 8 dims), so K and V come in as
// row-contiguous 16-byte loads, U steps of them in flight per wave; the G query
// heads of the kv head sit in registers.  A key's score is a DPP sum over its
// lanes (rows of 16 lanes, or half rows for DH 64); each lane keeps an online
// softmax (max and sum in base 2, its 8 output dims) per head over the keys of
// its lane row, rescaling once per batch of U keys; the workgroup's 4 * KPW row
// states are combined through LDS.  A sequence whose keys form one chunk gets
// its output written here; otherwise the chunk writes (max, sum) and the
// unnormalised output for attention_merge_kernel, with the chunk plan and the
// partial layout of attention_kernel.  Keys past the chunk's end read the
// chunk's last key (in bounds) and score -inf.
// ROPE: q points at the fp32 merged QKV rows and step A3 happens here too:
// wave 0 norms and rotates the G query rows of the stream's new token
// (rope_pairs, the arithmetic of qknorm_rope_kv_kernel, q rounded to fp16 as
// that kernel stores it) into LDS, and the workgroup of the last chunk also the new k row
// and the v row, writes both to the cache row start_pos and uses them from
// LDS for that key (its cache row is being written by the same launch).
struct RopeArgs {
  const void* qw;
  const void* kw;
  float theta, eps;
};

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int DH, int G, bool ROPE>
__global__ __launch_bounds__(256) void decode_attention_kernel(
    const void* __restrict__ q, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ start_pos, const int32_t* __restrict__ cache_slot,
    const int32_t* __restrict__ used_keys, int Hq, int Hkv, int cap, int causal, float scale_log2,
    void* __restrict__ out, int out_fp8, float out_inv, int chunk_tiles, int n_slots, float* __restrict__ part_o,
    float2_t* __restrict__ part_ml, int T, const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
    const RopeFreq freq, float eps) {
  constexpr int LPK = DH / 8;          // lanes per key
  constexpr int KPW = 64 / LPK;        // keys per wave instruction (lane rows)
  constexpr int KPS = 4 * KPW;         // keys per workgroup step
  constexpr int NR = 4 * KPW;          // row states per workgroup
  constexpr int U = 4;                 // steps per batch
  __shared__ float s_ml[G][NR][2];
  __shared__ float s_o[G][NR][DH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int t = cu[s];
  const int n_keys = causal ? start_pos[s] + 1 : used_keys[s];
  int ct, nch;
  chunk_plan((n_keys + AKT - 1) / AKT, chunk_tiles, n_slots, ct, nch);
  if (c >= nch) return;                                 // whole workgroup
  const int k0 = c * ct * AKT, k1 = min(n_keys, k0 + ct * AKT);
  const int r = lane / LPK, d8 = lane % LPK;
  const int R = wave * KPW + r;
  const size_t crow = size_t(cache_slot[s]) * cap;
  const int p_new = n_keys - 1;                          // ROPE: the new token's key

  __shared__ float s_cs[DH / 2], s_sn[DH / 2];
  __shared__ __attribute__((aligned(16))) uint16_t s_qr[ROPE ? G : 1][DH];
  __shared__ __attribute__((aligned(16))) uint16_t s_kn[ROPE ? DH : 8], s_vn[ROPE ? DH : 8];
  if constexpr (ROPE) {
    constexpr int HALF = DH / 2, L = DH / 16;            // rope layout: L lanes per head row
    const bool last = c == nch - 1;
    if (tid < HALF) rope_angle(p_new, freq.inv[tid], s_cs[tid], s_sn[tid]);
    __syncthreads();
    if (wave == 0) {
      const int row = lane / L, c8 = lane % L;
      const int n_rows = G + (last ? 2 : 0);
      const int rr = row < n_rows ? row : 0;             // spare lanes repeat row 0 (group_sum needs them)
      const int head = rr < G ? g * G + rr : (rr == G ? Hq + g : Hq + Hkv + g);
      const float* src = static_cast<const float*>(q) + (size_t(t) * (Hq + 2 * Hkv) + head) * DH;
      const F8 lo = load_f8(src + 8 * c8);
      const F8 hi = load_f8(src + HALF + 8 * c8);
      const uint16_t* nw = rr < G ? qw : kw;
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(nw + 8 * c8);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(nw + HALF + 8 * c8);
      const float ss = group_sum(pairs_sumsq(lo, hi), L);
      if (row < n_rows) {
        const size_t cdst = ((crow + p_new) * Hkv + g) * DH;
        if (rr <= G) {
          const float inv = 1.0f / __builtin_sqrtf(ss / float(DH) + eps);
          F8 r0, r1;
          rope_pairs(lo, hi, w0, w1, inv, &s_cs[8 * c8], &s_sn[8 * c8], r0, r1);
          const u32x4 o0 = rr < G ? pack8_f16(r0) : pack8_bf16(r0);
          const u32x4 o1 = rr < G ? pack8_f16(r1) : pack8_bf16(r1);
          uint16_t* dst = rr < G ? &s_qr[rr < G ? rr : 0][0] : &s_kn[0];
          *reinterpret_cast<u32x4*>(dst + 8 * c8) = o0;
          *reinterpret_cast<u32x4*>(dst + HALF + 8 * c8) = o1;
          if (rr == G) {
            *reinterpret_cast<u32x4*>(kc + cdst + 8 * c8) = o0;
            *reinterpret_cast<u32x4*>(kc + cdst + HALF + 8 * c8) = o1;
          }
        } else {
          const u32x4 v0 = pack8_bf16(lo), v1 = pack8_bf16(hi);
          *reinterpret_cast<u32x4*>(&s_vn[8 * c8]) = v0;
          *reinterpret_cast<u32x4*>(&s_vn[HALF + 8 * c8]) = v1;
          *reinterpret_cast<u32x4*>(vc + cdst + 8 * c8) = v0;
          *reinterpret_cast<u32x4*>(vc + cdst + HALF + 8 * c8) = v1;
        }
      }
    }
    __syncthreads();
  }

  float qf[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const u32x4 v = ROPE ? *reinterpret_cast<const u32x4*>(&s_qr[ROPE ? hh : 0][8 * d8])
                         : *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(q) +
                                                           (size_t(t) * Hq + g * G + hh) * DH + 8 * d8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[hh][e] = h_at(v, e);
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -__builtin_inff();
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }
  const int n_steps = (k1 - k0 + KPS - 1) / KPS;
  for (int s0 = 0; s0 < n_steps; s0 += U) {
    u32x4 kv[U], vv[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = k0 + (s0 + u) * KPS + wave * KPW + r;
      ok[u] = j < k1;
      const size_t row = (crow + (ok[u] ? j : k1 - 1)) * Hkv + g;
      kv[u] = *reinterpret_cast<const u32x4*>(kc + row * DH + 8 * d8);
      vv[u] = *reinterpret_cast<const u32x4*>(vc + row * DH + 8 * d8);
      if constexpr (ROPE) {
        // the new key: from LDS (the load above may race with its own write
        // and is discarded)
        if (j == p_new) {
          kv[u] = *reinterpret_cast<const u32x4*>(&s_kn[8 * d8]);
          vv[u] = *reinterpret_cast<const u32x4*>(&s_vn[8 * d8]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float x[U];
      float mb = -__builtin_inff();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += qf[hh][e] * ((e & 1) ? bf_hi(kv[u][e >> 1]) : bf_lo(kv[u][e >> 1]));
        dot = dpp_add<0xb1>(dot);                        // quad_perm [1,0,3,2]
        dot = dpp_add<0x4e>(dot);                        // quad_perm [2,3,0,1]
        dot = dpp_add<0x141>(dot);                       // row_half_mirror: 8 lanes
        if constexpr (LPK == 16) dot = dpp_add<0x140>(dot);   // row_mirror: 16 lanes
        x[u] = ok[u] ? dot * scale_log2 : -__builtin_inff();
        mb = fmaxf(mb, x[u]);
      }
      const float mn = fmaxf(m[hh], mb);
      if (mn == -__builtin_inff()) continue;             // nothing unmasked yet in this lane row
      const float sc = __builtin_amdgcn_exp2f(m[hh] - mn);   // 0 when m was -inf
      l[hh] *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] *= sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = __builtin_amdgcn_exp2f(x[u] - mn);   // 0 for masked keys
        l[hh] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] += p * ((e & 1) ? bf_hi(vv[u][e >> 1]) : bf_lo(vv[u][e >> 1]));
      }
      m[hh] = mn;
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    if (d8 == 0) {
      s_ml[hh][R][0] = m[hh];
      s_ml[hh][R][1] = l[hh];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_o[hh][R][8 * d8 + e] = o[hh][e];
  }
  __syncthreads();
  for (int u = tid; u < G * DH; u += 256) {
    const int hh = u / DH, d = u % DH;
    float M = -__builtin_inff();
    for (int i = 0; i < NR; ++i) M = fmaxf(M, s_ml[hh][i][0]);
    float L = 0.f, O = 0.f;
    for (int i = 0; i < NR; ++i) {
      const float mi = s_ml[hh][i][0];
      const float w = mi == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mi - M);
      L += w * s_ml[hh][i][1];
      O += w * s_o[hh][i][d];
    }
    const int hq = g * G + hh;
    if (nch == 1) {
      const float y = O / L;
      const size_t orow = (size_t(t) * Hq + hq) * DH + d;
      if (out_fp8) static_cast<uint8_t*>(out)[orow] = uint8_t(f2e4m3(y * out_inv));
      else static_cast<uint16_t*>(out)[orow] = uint16_t(f2h(y));
    } else {
      const size_t prow = (size_t(c) * T + t) * Hq + hq;
      part_o[prow * DH + d] = O;
      if (d == 0) part_ml[prow] = float2_t{M, L};
    }
  }
}

template <int DH, int GROUP>
static void launch_decode_t(const void* q, const void* kc, const void* vc, const int32_t* cu, const int32_t* sp,
                            const int32_t* slot, const int32_t* used, int n_seq, int Hq, int Hkv, int cap,
                            bool causal, void* out, bool fp8, float out_inv, const AttnSplit& cfg, hipStream_t st,
                            const RopeArgs* rope = nullptr) {
  const int slots = cfg.chunk_tiles > 0 ? cfg.n_slots : 1;
  const dim3 grid(slots, Hkv, n_seq);
  const float scale_log2 = 1.4426950408889634f / __builtin_sqrtf(float(DH));
  // kc and vc are written only on the RoPE path (the new token's row)
  uint16_t* kcw = static_cast<uint16_t*>(const_cast<void*>(kc));
  uint16_t* vcw = static_cast<uint16_t*>(const_cast<void*>(vc));
  if (rope)
    decode_attention_kernel<DH, GROUP, true><<<grid, 256, 0, st>>>(
        q, kcw, vcw, cu, sp, slot, used, Hq, Hkv, cap, causal ? 1 : 0, scale_log2,
        out, fp8 ? 1 : 0, out_inv, cfg.chunk_tiles, slots, cfg.part_o, reinterpret_cast<float2_t*>(cfg.part_ml),
        cfg.T, static_cast<const uint16_t*>(rope->qw), static_cast<const uint16_t*>(rope->kw),
        rope_freq(DH, rope->theta), rope->eps);
  else
    decode_attention_kernel<DH, GROUP, false><<<grid, 256, 0, st>>>(
        q, kcw, vcw, cu, sp, slot, used, Hq, Hkv, cap, causal ? 1 : 0, scale_log2,
        out, fp8 ? 1 : 0, out_inv, cfg.chunk_tiles, slots, cfg.part_o, reinterpret_cast<float2_t*>(cfg.part_ml),
        cfg.T, nullptr, nullptr, RopeFreq{}, 0.f);
  if (cfg.chunk_tiles > 0)
    attention_merge_kernel<DH><<<dim3(cfg.T, (Hq * (DH / 4) + 255) / 256), 256, 0, st>>>(
        cu, sp, used, n_seq, Hq, causal ? 1 : 0, 1, cfg.chunk_tiles,
                                                      slots, cfg.part_o,
                                                      reinterpret_cast<const float2_t*>(cfg.part_ml), cfg.T, out,
                                                      fp8 ? 1 : 0, out_inv);
}

template <int DH, int GROUP>
static void launch_attn_t(const void* q, const void* kc, const void* vc, const int32_t* cu,
                          const int32_t* sp, const int32_t* slot, const int32_t* used, int n_seq,
                          int max_len, int Hq, int Hkv, int cap, bool causal, void* out, bool fp8,
                          float out_inv, const AttnSplit& sp_cfg, hipStream_t st) {
  constexpr int QPW = 32 * (4 / GROUP);
  const int n_qb = (max_len + QPW - 1) / QPW;
  const int slots = sp_cfg.chunk_tiles > 0 ? sp_cfg.n_slots : 1;
  // head split only where the group divides (GROUP 2 and 4)
  const int hsplit = (sp_cfg.head_split == 2 && GROUP % 2 == 0) ? 2 : 1;
  dim3 grid(n_qb * slots, Hkv * hsplit, n_seq);
  const float scale_log2 = 1.4426950408889634f / __builtin_sqrtf(float(DH));
#define HR_ATT_LAUNCH(NG_, HS_)                                                                  \
  attention_kernel<DH, GROUP, NG_, HS_><<<grid, 64 * (GROUP / HS_) * (4 / GROUP) * NG_, 0, st>>>( \
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),                         \
      static_cast<const uint16_t*>(vc), cu, sp, slot, used, Hq, Hkv, cap, causal ? 1 : 0,        \
      scale_log2, out, fp8 ? 1 : 0, out_inv, sp_cfg.chunk_tiles, slots, sp_cfg.part_o,          \
      reinterpret_cast<float2_t*>(sp_cfg.part_ml), sp_cfg.T)
  if constexpr (GROUP % 2 == 0) {
    if (hsplit == 2) {
      if (sp_cfg.groups == 2) HR_ATT_LAUNCH(2, 2);
      else HR_ATT_LAUNCH(1, 2);
    } else if (sp_cfg.groups == 2) {
      HR_ATT_LAUNCH(2, 1);
    } else {
      HR_ATT_LAUNCH(1, 1);
    }
  } else {
    if (sp_cfg.groups == 2) HR_ATT_LAUNCH(2, 1);
    else HR_ATT_LAUNCH(1, 1);
  }
#undef HR_ATT_LAUNCH
  if (sp_cfg.chunk_tiles > 0)
    attention_merge_kernel<DH><<<dim3(sp_cfg.T, (Hq * (DH / 4) + 255) / 256), 256, 0, st>>>(
        cu, sp, used, n_seq, Hq, causal ? 1 : 0, QPW,
                                                         sp_cfg.chunk_tiles, slots, sp_cfg.part_o,
                                                         reinterpret_cast<const float2_t*>(sp_cfg.part_ml),
                                                         sp_cfg.T, out, fp8 ? 1 : 0, out_inv);
}

int attention_qpw(int Hq, int Hkv) { return 32 * (4 / (Hq / Hkv)); }

template <int DH>
static void attention_f16_go(const dim3& grid, const void* q, const void* k16, const void* v16, int Tp,
                             const int32_t* cu, const int32_t* used, int Hq, int Hkv, bool causal, float scale_log2,
                             void* out, bool fp8, float out_inv, hipStream_t st) {
  constexpr size_t kLds = attention_f16_lds<DH>();
  auto kern = attention_f16_kernel<DH>;
  if (kLds > 65536) {
    // above the 64 KB default dynamic-LDS limit: raised once (a thread-safe
    // static); a refusal surfaces as the launch's error
    static const hipError_t raised = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(kLds));
    (void)raised;
  }
  kern<<<grid, 64 * kF16Waves, kLds, st>>>(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k16),
                                           static_cast<const uint16_t*>(v16), Tp, cu, used, Hq, Hkv, causal ? 1 : 0,
                                           scale_log2, out, fp8 ? 1 : 0, out_inv);
}

void launch_attention_f16(const void* q, const void* k16, const void* v16, int Tp, const int32_t* cu,
                          const int32_t* used, int n_seq, int max_len, int Hq, int Hkv, int d, bool causal,
                          void* out, bool fp8, float out_inv, hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / __builtin_sqrtf(float(d));
  const int nb = (max_len + 31) / 32;
  const dim3 grid((nb + 1) / 2, Hq, n_seq);
  if (d == 128)
    attention_f16_go<128>(grid, q, k16, v16, Tp, cu, used, Hq, Hkv, causal, scale_log2, out, fp8, out_inv, st);
  else
    attention_f16_go<64>(grid, q, k16, v16, Tp, cu, used, Hq, Hkv, causal, scale_log2, out, fp8, out_inv, st);
}

void launch_decode_rope_attention(const void* qkv, const void* qw, const void* kw, float theta, float eps,
                                  void* kc, void* vc, const int32_t* cu, const int32_t* sp, const int32_t* slot,
                                  int n_seq, int Hq, int Hkv, int d, int cap, void* out, bool fp8, float out_inv,
                                  const AttnSplit& cfg, hipStream_t st) {
  const int group = Hq / Hkv;
  const RopeArgs rope{qw, kw, theta, eps};
#define HR_DEC(DH_, G_)                                                                         \
  if (d == DH_ && group == G_) {                                                                \
    launch_decode_t<DH_, G_>(qkv, kc, vc, cu, sp, slot, nullptr, n_seq, Hq, Hkv, cap, true, out, \
                             fp8, out_inv, cfg, st, &rope);                                     \
    return;                                                                                     \
  }
  HR_DEC(128, 4) HR_DEC(128, 2) HR_DEC(128, 1) HR_DEC(64, 4) HR_DEC(64, 2) HR_DEC(64, 1)
#undef HR_DEC
}

void launch_attention(const void* q, const void* kc, const void* vc, const int32_t* cu,
                      const int32_t* sp, const int32_t* slot, const int32_t* used, int n_seq,
                      int max_len, int Hq, int Hkv, int d, int cap, bool causal, void* out, bool fp8,
                      float out_inv, hipStream_t st, const AttnSplit* split) {
  const int group = Hq / Hkv;
  const AttnSplit none{};
  const AttnSplit& cfg = split ? *split : none;
#define HR_ATT(DH_, G_)                                                                         \
  if (d == DH_ && group == G_) {                                                                \
    if (cfg.decode)                                                                             \
      launch_decode_t<DH_, G_>(q, kc, vc, cu, sp, slot, used, n_seq, Hq, Hkv, cap, causal, out, \
                               fp8, out_inv, cfg, st);                                          \
    else                                                                                        \
      launch_attn_t<DH_, G_>(q, kc, vc, cu, sp, slot, used, n_seq, max_len, Hq, Hkv, cap,       \
                             causal, out, fp8, out_inv, cfg, st);                               \
    return;                                                                                     \
  }
  HR_ATT(128, 4) HR_ATT(128, 2) HR_ATT(128, 1) HR_ATT(64, 4) HR_ATT(64, 2) HR_ATT(64, 1)
#undef HR_ATT
}

}  // namespace hr
