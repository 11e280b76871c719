// Partition-phase kernel for the [num_blocks, Hkv, block_size, head_size]
// cache layout (the dispatch page's decode signature: key and value caches
// of shape (num_blocks, num_kv_heads, block_size, head_dim)), 16-bit caches.
//
// A (block, KV head) tile is block_size rows of head_size contiguous
// elements, for K and for V alike.  Load i of lane l reads bytes
// [1024 i + 16 l, +16): token TPL i + l / R (R = head_size / 8 lanes per
// row), dims 8 c .. 8 c + 7 with c = l % R -- one fixed 8-dim chunk per lane,
// so each lane keeps just that chunk of every query head.
//   q.K: four dot2 per head and load, summed over the R lanes of the row.
//   P.V: for loads 2j and 2j + 1 (two tokens, the same dims) a byte permute
//        pairs each dim's two values and one dot2 per dim and head adds both
//        tokens' weighted values; the sums over the lanes' tokens are
//        combined across the token groups at the end.
// Work decoding, masks, window, soft cap, ALiBi, poisoning and the epilogue
// are those of the other partition kernels.
#pragma once

#include "pa_launch.h"
#include "pa_partition_common.h"

namespace pa {

// Sum over the R lanes of a token row (R = 16: a DPP row; R = 8: half a row).
template <int R>
__device__ __forceinline__ float row_group_sum(float v) {
  v += dpp<0xB1>(v);  // xor 1
  v += dpp<0x4E>(v);  // xor 2
  v += __shfl_xor(v, 4);
  if constexpr (R == 16) v += dpp<0x128>(v);  // row_ror:8
  return v;
}

// Max / sum over the token groups of a wave (lanes l, l ^ R, l ^ 2R, ...).
template <int R>
__device__ __forceinline__ float token_groups_max(float v) {
  if constexpr (R == 8) v = fmaxf(v, __shfl_xor(v, 8));
  return xor_max<32>(xor_max<16>(v));
}
template <int R>
__device__ __forceinline__ float token_groups_sum(float v) {
  if constexpr (R == 8) v += __shfl_xor(v, 8);
  return xor_sum<32>(xor_sum<16>(v));
}

template <typename QT, int D, int BS, int GP, bool CAP, bool WIN>
__global__ void __launch_bounds__(kThreads) pa_partition_nhd(const Params p) {
  constexpr int R = D / 8;                  // lanes per token row
  constexpr int TPL = 64 / R;               // tokens per 1 KB load
  constexpr int TILE = BS * D * 2;          // bytes of one (block, KV head) K or V tile
  constexpr int NL = TILE / 1024;           // 16-byte loads per lane per tile
  static_assert(NL >= 2 && NL % 2 == 0 && NL * 1024 == TILE, "tile geometry");
  static_assert(GP <= nhd_max_group(D, BS), "head group too wide for the registers");

  __shared__ float sm_o[kWaves][GP][D];
  __shared__ float sm_m[kWaves][GP];
  __shared__ float sm_l[kWaves][GP];

  Work w;
  if (!begin_work<QT, D>(p, BS, GP, w)) return;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane % R;       // this lane's 8-dim chunk
  const int tgrp = lane / R;    // token group: token TPL i + tgrp of load i

  // The lane's chunk of every head's query (4 packed 16-bit pairs).
  unsigned qw[GP][4];
  float slope2[GP];
  {
    const QT *qbase = reinterpret_cast<const QT *>(p.query) +
                      ((size_t)w.seq * p.num_heads + w.head0) * D + 8 * c;
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const u32x4 v = h < w.nh ? load16(qbase + h * D) : u32x4{0u, 0u, 0u, 0u};
      qw[h][0] = v.x; qw[h][1] = v.y; qw[h][2] = v.z; qw[h][3] = v.w;
      slope2[h] = (p.alibi_slopes && h < w.nh) ? p.alibi_slopes[w.head0 + h] * kLog2e : 0.0f;
    }
  }

  float m_run[GP], l_run[GP], acc[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    m_run[h] = -__builtin_inff();
    l_run[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }

  const char *kcache = reinterpret_cast<const char *>(p.key_cache);
  const char *vcache = reinterpret_cast<const char *>(p.value_cache);
  const const_i32_ptr btab = as_const_table(p.block_tables + (size_t)w.seq * p.max_num_blocks_per_seq);
  const size_t head_off = (size_t)w.kvh * TILE;
  const size_t blk_stride = (size_t)p.num_kv_heads * TILE;
  bool poisoned = false;

  struct Tile {
    u32x4 k[NL], v[NL];
  };
  // Out-of-range block-table entries read block 0 and poison the result.
  auto load_tile = [&](int blk) {
    int phys = btab[blk];
    if (phys < 0 || phys >= p.num_blocks) {
      poisoned = true;
      phys = 0;
    }
    const char *kb = kcache + (size_t)phys * blk_stride + head_off + 16 * lane;
    const char *vb = vcache + (size_t)phys * blk_stride + head_off + 16 * lane;
    Tile t;
#pragma unroll
    for (int i = 0; i < NL; ++i) t.k[i] = load16_stream(kb + 1024 * i);
#pragma unroll
    for (int i = 0; i < NL; ++i) t.v[i] = load16_stream(vb + 1024 * i);
    return t;
  };

  auto process = [&](int blk, const Tile &tl) {
    const int t0 = blk * BS + tgrp;  // token of load 0; load i adds TPL i
    // Logits of this lane's NL tokens for every head.
    float x[GP][NL];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float s = 0.0f;
        s = dot2(s, qw[h][0], tl.k[i].x, QT());
        s = dot2(s, qw[h][1], tl.k[i].y, QT());
        s = dot2(s, qw[h][2], tl.k[i].z, QT());
        s = dot2(s, qw[h][3], tl.k[i].w, QT());
        s = row_group_sum<R>(s);
        const int t = t0 + TPL * i;
        const float v = scaled_logit<CAP>(p, s) + slope2[h] * (float)(t - w.t_ref);
        x[h][i] = in_span<WIN>(t, w.t_lo, w.span) ? v : -__builtin_inff();
      }
    // V of tokens outside the window / past the end is zeroed (never NaN).
    u32x4 vv[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i)
      vv[i] = in_span<WIN>(t0 + TPL * i, w.t_lo, w.span) ? tl.v[i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float bm = x[h][0];
#pragma unroll
      for (int i = 1; i < NL; ++i) bm = fmaxf(bm, x[h][i]);
      bm = token_groups_max<R>(bm);
      const float m_new = fmaxf(m_run[h], bm);
      const float alpha = (m_new == -__builtin_inff()) ? 1.0f : fast_exp2(m_run[h] - m_new);
      m_run[h] = m_new;
      float pe[NL], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        pe[i] = x[h][i] == -__builtin_inff() ? 0.0f : fast_exp2(x[h][i] - m_new);
        psum += pe[i];
      }
      l_run[h] = l_run[h] * alpha + psum;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int j = 0; j < NL / 2; ++j) {
        const unsigned pp = pack2(pe[2 * j], pe[2 * j + 1], QT());
        const unsigned a[4] = {vv[2 * j].x, vv[2 * j].y, vv[2 * j].z, vv[2 * j].w};
        const unsigned b[4] = {vv[2 * j + 1].x, vv[2 * j + 1].y, vv[2 * j + 1].z, vv[2 * j + 1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // Dim e of the two tokens as one packed pair (low half: token 2j).
          const unsigned vp =
              __builtin_amdgcn_perm(b[e / 2], a[e / 2], (e % 2) ? 0x07060302u : 0x05040100u);
          acc[h][e] = dot2(acc[h][e], pp, vp, QT());
        }
      }
    }
  };

  // Two tiles ping-pong, as in the other partition kernels: the loop runs
  // whole pairs with no exit between them and always issues its loads.
  int blk = w.blk_begin + wv;
  int left = blk < w.blk_end ? (w.blk_end - blk + kWaves - 1) / kWaves : 0;
  Tile ta, tb;
  if (left > 0) ta = load_tile(blk);
  while (left >= 3) {
    tb = load_tile(blk + kWaves);
    __builtin_amdgcn_sched_barrier(0);
    process(blk, ta);
    ta = load_tile(blk + 2 * kWaves);
    __builtin_amdgcn_sched_barrier(0);
    process(blk + kWaves, tb);
    blk += 2 * kWaves;
    left -= 2;
  }
  if (left == 2) {
    tb = load_tile(blk + kWaves);
    __builtin_amdgcn_sched_barrier(0);
    process(blk, ta);
    process(blk + kWaves, tb);
  } else if (left == 1) {
    process(blk, ta);
  }

  // Wave totals: sums over the token groups (the R lanes of a row hold the
  // same token weights, so only the groups are summed).
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    const float l_tot = token_groups_sum<R>(l_run[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = token_groups_sum<R>(acc[h][e]);
    if (tgrp == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wv][h][8 * c + e] = acc[h][e];
    }
    if (lane == 0) {
      sm_m[wv][h] = m_run[h];
      sm_l[wv][h] = poisoned ? __builtin_nanf("") : l_tot;
    }
  }
  __syncthreads();
  finish_partition<QT, D, GP, D>(p, w, sm_o, sm_m, sm_l);
}

}  // namespace pa
