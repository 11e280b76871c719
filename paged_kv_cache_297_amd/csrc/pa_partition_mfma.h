// Partition-phase kernel, MFMA form: for GQA groups wide enough (5..16 query
// heads per KV head) that QK^T and PV become real dense 16-row tiles.
//
// A (block, KV head) tile is processed as bs/16 sub-tiles of 16 tokens.
//   S^T = K . Q^T  with v_mfma_f32_16x16x32 (bf16/f16): A = 16 tokens x 32
//        dims of K, B = 32 dims x 16 query heads (the group, zero padded).
//        Lane l feeds token l%16 with the 16-byte K chunk 4i + l/16 of load i,
//        which is exactly the coalesced 1 KB-per-instruction read of the
//        [D/x][bs][x] layout (fp8 chunks hold 16 dims and feed two k-steps;
//        the query slices follow the same dim order).
//   O^T += V^T . P^T with v_mfma_f32_16x16x16: the S^T accumulator leaves
//        lane l with head l%16 and tokens 4(l/16)..+3, which is the B operand
//        layout of the 16x16x16 MFMA, so P never leaves registers; A = 16 dims
//        x 16 tokens of V, read as 4 consecutive tokens of one dim per lane
//        (8 bytes for 16-bit V, 4 for fp8) -- 512 / 256 contiguous bytes per
//        wave instruction.
// Each lane keeps the running max / sum of one query head (l%16), so the
// online-softmax rescale of O needs no broadcast.  fp8 E4M3FN keys are
// widened exactly to the query's 16-bit type, values to fp16 (P in fp16).
#pragma once

#include <type_traits>

#include "pa_partition_common.h"

namespace pa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_qk(const u32x4 &a, const u32x4 &b, const f32x4 &c,
                                         __bf16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_qk(const u32x4 &a, const u32x4 &b, const f32x4 &c,
                                         _Float16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_pv(const u32x2 &a, const u32x2 &b, const f32x4 &c,
                                         __bf16) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_pv(const u32x2 &a, const u32x2 &b, const f32x4 &c,
                                         _Float16) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                               __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Zero the 16-bit elements of tokens >= nv in a 4-token V operand.
__device__ __forceinline__ u32x2 mask_v4(u32x2 v, int first, int nv) {
  if (first >= nv) v.x = 0u;
  else if (first + 1 >= nv) v.x &= 0xFFFFu;
  if (first + 2 >= nv) v.y = 0u;
  else if (first + 3 >= nv) v.y &= 0xFFFFu;
  return v;
}

template <typename QT, typename KVT, int D, int BS>
__global__ void __launch_bounds__(kThreads) pa_partition_mfma(const Params p) {
  constexpr bool kFp8 = std::is_same<KVT, fp8e4m3>::value;
  using PT = typename std::conditional<kFp8, _Float16, KVT>::type;  // P.V operand type
  static_assert(kFp8 || std::is_same<KVT, QT>::value, "16-bit cache must match the query type");
  constexpr int ESZ = kFp8 ? 1 : 2;
  constexpr int NSUB = BS / 16;               // 16-token sub-tiles per block
  constexpr int TILE = D * BS * ESZ;          // bytes of one K or V tile
  constexpr int NLK = D * 16 * ESZ / 1024;    // 16-byte K loads per lane per sub-tile
  constexpr int NKS = D / 32;                 // 32-dim k-steps of QK
  constexpr int NDT = D / 16;                 // 16-dim tiles of the output
  constexpr int OSTR = D + 4;                 // padded LDS row (bank spread)
  static_assert(NLK >= 1 && NLK * (kFp8 ? 2 : 1) == NKS, "K sub-tile geometry");

  __shared__ float sm_o[kWaves][16][OSTR];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];

  Work w;
  if (!begin_work<QT, D>(p, BS, 16, w)) return;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;   // query head of the group (MFMA column)
  const int g = lane >> 4;   // lane group: k-slot block / row block

  // B operands of QK: 8 query values per lane and k-step, in the dim order
  // of the K chunks (16-bit: dims 32ks + 8g + e; fp8: chunk 4i + g of 16 dims,
  // halves ks = 2i and 2i + 1).
  u32x4 qop[NKS];
  {
    const QT *q = reinterpret_cast<const QT *>(p.query) +
                  ((size_t)w.seq * p.num_heads + w.head0 + n) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int dim0 = kFp8 ? (16 * (4 * (ks / 2) + g) + 8 * (ks % 2)) : (32 * ks + 8 * g);
      qop[ks] = (n < w.nh) ? load16(q + dim0) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const float slope2 = (p.alibi_slopes && n < w.nh) ? p.alibi_slopes[w.head0 + n] * kLog2e : 0.0f;

  float m_run = -__builtin_inff(), l_run = 0.0f;
  f32x4 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const char *kcache = reinterpret_cast<const char *>(p.key_cache);
  const char *vcache = reinterpret_cast<const char *>(p.value_cache);
  const int32_t *btab = p.block_tables + (size_t)w.seq * p.max_num_blocks_per_seq;
  const size_t head_off = (size_t)w.kvh * TILE;
  const size_t blk_stride = (size_t)p.num_kv_heads * TILE;
  bool poisoned = false;

  // K: sub-tile s, load i -> chunk 4i + g, token 16s + n.
  // V: sub-tile s, dim tile t -> dim 16t + n, tokens 16s + 4g .. +3.
  struct Tile {
    u32x4 k[NSUB][NLK];
    typename std::conditional<kFp8, unsigned, u32x2>::type v[NSUB][NDT];
  };

  // Out-of-range block-table entries are redirected to block 0 (always
  // addressable) and reported through the poison flag.
  auto load_tile = [&](int blk) {
    int phys = btab[blk];
    if (phys < 0 || phys >= p.num_blocks) {
      poisoned = true;
      phys = 0;
    }
    const char *kb = kcache + (size_t)phys * blk_stride + head_off;
    const char *vb = vcache + (size_t)phys * blk_stride + head_off;
    Tile tl;
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int i = 0; i < NLK; ++i)
        tl.k[s][i] = load16_stream(kb + (4 * i + g) * (BS * 16) + (16 * s + n) * 16);
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const char *src = vb + ((16 * t + n) * BS + 16 * s + 4 * g) * ESZ;
        if constexpr (kFp8) tl.v[s][t] = load4_stream(src);
        else tl.v[s][t] = load8_stream(src);
      }
    return tl;
  };

  auto process = [&](int blk, const Tile &tl) {
    // S^T for each 16-token sub-tile: lane holds head n, tokens 16s + 4g + e.
    f32x4 st[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < NLK; ++i) {
        if constexpr (kFp8) {
          const u32x4 kw = tl.k[s][i];
          const u32x4 lo = {fp8x2_to<false>(kw.x, QT()), fp8x2_to<true>(kw.x, QT()),
                            fp8x2_to<false>(kw.y, QT()), fp8x2_to<true>(kw.y, QT())};
          const u32x4 hi = {fp8x2_to<false>(kw.z, QT()), fp8x2_to<true>(kw.z, QT()),
                            fp8x2_to<false>(kw.w, QT()), fp8x2_to<true>(kw.w, QT())};
          c = mfma_qk(lo, qop[2 * i], c, QT());
          c = mfma_qk(hi, qop[2 * i + 1], c, QT());
        } else {
          c = mfma_qk(tl.k[s][i], qop[i], c, QT());
        }
      }
      st[s] = c;
    }
    // Scale, ALiBi, mask, block max over the head's tokens.
    const int t0 = blk * BS;
    float x[NSUB][4];
    float bm = -__builtin_inff();
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 16 * s + 4 * g + e;
        float v = st[s][e] * p.scale_log2 + slope2 * (float)(t - w.t_ref);
        v = (t < w.L) ? v : -__builtin_inff();
        x[s][e] = v;
        bm = fmaxf(bm, v);
      }
    bm = xor_max<32>(xor_max<16>(bm));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = (m_new == -__builtin_inff()) ? 1.0f : fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.0f;
    u32x2 pop[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = fast_exp2(x[s][e] - m_new);
        psum += pe[e];
      }
      pop[s] = u32x2{pack2(pe[0], pe[1], PT()), pack2(pe[2], pe[3], PT())};
    }
    l_run = l_run * alpha + psum;
    const int nv = w.L - t0;  // valid tokens in the block (>= 1)
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      f32x4 c = oacc[t] * alpha;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        u32x2 va;
        if constexpr (kFp8) {
          va = u32x2{fp8x2_to<false>(tl.v[s][t], _Float16()), fp8x2_to<true>(tl.v[s][t], _Float16())};
        } else {
          va = tl.v[s][t];
        }
        if (nv < BS) va = mask_v4(va, 16 * s + 4 * g, nv);
        c = mfma_pv(va, pop[s], c, PT());
      }
      oacc[t] = c;
    }
  };

  // Two tiles in flight: the next block's loads are issued before the
  // current block is consumed (ping-pong, no register copies).
  int blk = w.blk_begin + wv;
  Tile ta, tb;
  if (blk < w.blk_end) ta = load_tile(blk);
  while (blk < w.blk_end) {
    if (blk + kWaves < w.blk_end) tb = load_tile(blk + kWaves);
    process(blk, ta);
    blk += kWaves;
    if (blk >= w.blk_end) break;
    if (blk + kWaves < w.blk_end) ta = load_tile(blk + kWaves);
    process(blk, tb);
    blk += kWaves;
  }

  // Wave totals: the four lanes of head n hold partial sums over their tokens.
  const float l_tot = xor_sum<32>(xor_sum<16>(l_run));
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) sm_o[wv][n][16 * t + 4 * g + e] = oacc[t][e];
  if (g == 0) {
    sm_m[wv][n] = m_run;
    sm_l[wv][n] = poisoned ? __builtin_nanf("") : l_tot;
  }
  __syncthreads();
  finish_partition<QT, D, 16, OSTR>(p, w, sm_o, sm_m, sm_l);
}

}  // namespace pa
