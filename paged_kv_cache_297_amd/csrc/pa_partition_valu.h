// Partition-phase kernel, VALU form: for narrow GQA groups (and fp32), where
// a 16-row MFMA tile would be mostly padding.
//
// Per (block, KV head) tile the wave issues NL coalesced 16-byte loads per
// lane for K and NL for V: load i of lane l reads bytes [1024 i + 16 l,
// +16) of the tile, so every wave instruction reads 1 KB of contiguous
// memory (the lesson of the Neuron vectorised-KV-load PR: the paged gather is
// bound by HBM fetch, so fetch whole tiles with wide loads).  In the K layout
// [D/x][bs][x] that hands lane l token (l % bs) and 16-byte chunk
// (i * 64/bs + l / bs); the 64/bs lanes that share a token combine their
// partial dot products with permlane swaps that also transpose, so that
// afterwards each lane holds whole logits for max(1, GP*bs/64) query heads.
// The GQA group's query slices stay in registers for the whole workgroup.
//
// Softmax is online per wave (running max / sum in log2 units); P is passed
// to the V layout through a small per-wave LDS buffer, rounded to the V
// element type as the V2 page does before its weighted sum.
#pragma once

#include <type_traits>

#include "pa_partition_common.h"

namespace pa {

// Per (query type, KV storage type): how 16-byte K chunks meet the query and
// how 16-byte V units meet P.
template <typename QT, typename KVT>
struct ValuTraits;

template <>
struct ValuTraits<float, float> {
  static constexpr int kBytes = 4;  // storage bytes per KV element
  static constexpr int kQW = 4;     // 32-bit query words per 16-byte K chunk
  static constexpr int kPW = 4;     // 32-bit P words per 16-byte V unit
  using PV = float;                 // type P is rounded to before P.V
  __device__ static void load_q(const float *q, unsigned (&w)[kQW]) {
    const u32x4 v = load16(q);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  __device__ static float qk(float acc, const unsigned (&q)[kQW], const u32x4 &k) {
    acc = fmaf(bits_f(q[0]), bits_f(k.x), acc);
    acc = fmaf(bits_f(q[1]), bits_f(k.y), acc);
    acc = fmaf(bits_f(q[2]), bits_f(k.z), acc);
    acc = fmaf(bits_f(q[3]), bits_f(k.w), acc);
    return acc;
  }
  __device__ static void v_words(const u32x4 &v, unsigned (&w)[kPW]) {
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  __device__ static float pv(float acc, const unsigned (&pw)[kPW], const unsigned (&vw)[kPW]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(bits_f(pw[e]), bits_f(vw[e]), acc);
    return acc;
  }
  // Zero the V elements of tokens outside [lo, lo + span) (first = token of
  // element 0).
  template <bool WIN>
  __device__ static void mask_v(unsigned (&w)[kPW], int first, int lo, int span) {
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] &= in_span<WIN>(first + e, lo, span) ? ~0u : 0u;
  }
};

template <typename T16>
struct ValuTraits16 {
  static constexpr int kBytes = 2;
  static constexpr int kQW = 4;
  static constexpr int kPW = 4;
  using PV = T16;
  __device__ static void load_q(const T16 *q, unsigned (&w)[kQW]) {
    const u32x4 v = load16(q);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  __device__ static float qk(float acc, const unsigned (&q)[kQW], const u32x4 &k) {
    acc = dot2(acc, q[0], k.x, T16());
    acc = dot2(acc, q[1], k.y, T16());
    acc = dot2(acc, q[2], k.z, T16());
    acc = dot2(acc, q[3], k.w, T16());
    return acc;
  }
  __device__ static void v_words(const u32x4 &v, unsigned (&w)[kPW]) {
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  __device__ static float pv(float acc, const unsigned (&pw)[kPW], const unsigned (&vw)[kPW]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = dot2(acc, pw[e], vw[e], T16());
    return acc;
  }
  template <bool WIN>
  __device__ static void mask_v(unsigned (&w)[kPW], int first, int lo, int span) {
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] &= keep_pair_mask<WIN>(first + 2 * e, lo, span);
  }
};
template <> struct ValuTraits<__bf16, __bf16> : ValuTraits16<__bf16> {};
template <> struct ValuTraits<_Float16, _Float16> : ValuTraits16<_Float16> {};

// fp8 E4M3FN cache: K is widened exactly to the query's 16-bit type for the
// dot products, V to fp16 (exact for every E4M3 value) with P in fp16.
template <typename T16>
struct ValuTraitsFp8 {
  static constexpr int kBytes = 1;
  static constexpr int kQW = 8;   // 16 fp8 dims per chunk -> 8 packed pairs
  static constexpr int kPW = 8;   // 16 fp8 tokens per V unit -> 8 fp16 pairs
  using PV = _Float16;
  __device__ static void load_q(const T16 *q, unsigned (&w)[kQW]) {
    const u32x4 a = load16(q), b = load16(q + 8);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  __device__ static float qk(float acc, const unsigned (&q)[kQW], const u32x4 &k) {
    const unsigned kw[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = dot2(acc, q[2 * e], fp8x2_to<false>(kw[e], T16()), T16());
      acc = dot2(acc, q[2 * e + 1], fp8x2_to<true>(kw[e], T16()), T16());
    }
    return acc;
  }
  __device__ static void v_words(const u32x4 &v, unsigned (&w)[kPW]) {
    const unsigned vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[2 * e] = fp8x2_to<false>(vw[e], _Float16());
      w[2 * e + 1] = fp8x2_to<true>(vw[e], _Float16());
    }
  }
  __device__ static float pv(float acc, const unsigned (&pw)[kPW], const unsigned (&vw)[kPW]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = dot2(acc, pw[e], vw[e], _Float16());
    return acc;
  }
  // Applied to the widened words: word e holds tokens first+2e, first+2e+1.
  template <bool WIN>
  __device__ static void mask_v(unsigned (&w)[kPW], int first, int lo, int span) {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] &= keep_pair_mask<WIN>(first + 2 * e, lo, span);
  }
};
template <> struct ValuTraits<__bf16, fp8e4m3> : ValuTraitsFp8<__bf16> {};
template <> struct ValuTraits<_Float16, fp8e4m3> : ValuTraitsFp8<_Float16> {};

// Which query heads a lane holds after the transpose-reduce over the R = 64/bs
// lanes of a token: lane group r = lane / bs holds heads head_base(r) ..
// head_base(r) + NF - 1.  Each reduce step over lane bit (bs << b) halves the
// set of heads a lane carries while it is >= 2, keeping the upper half when
// the bit is set (the permlane swap pairing above).
template <int GP, int BS>
struct HeadMap {
  static constexpr int R = 64 / BS;
  static constexpr int NF = GP >= R ? GP / R : 1;
  static constexpr int head_base(int r) {
    int h = 0, n = GP, b = 0;
    for (int m = BS; m < 64; m *= 2, ++b) {
      if (n >= 2) {
        h += ((r >> b) & 1) * (n / 2);
        n /= 2;
      }
    }
    return h;
  }
  static constexpr int src_group(int h) {
    for (int r = 0; r < R; ++r)
      if (head_base(r) <= h && h < head_base(r) + NF) return r;
    return 0;
  }
};

template <int M, int N>
__device__ __forceinline__ void xreduce_step(float *v) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
      float a, b;
      swap_pair<M>(v[j], v[N / 2 + j], a, b);
      v[j] = a + b;
    }
  } else {
    v[0] = xor_sum<M>(v[0]);
  }
}

template <int GP, int BS>
__device__ __forceinline__ void transpose_reduce(float (&v)[GP]) {
  if constexpr (BS == 16) {
    xreduce_step<16, GP>(v);
    xreduce_step<32, (GP >= 2 ? GP / 2 : 1)>(v);
  } else {
    xreduce_step<32, GP>(v);
  }
}

template <int BS>
__device__ __forceinline__ float token_group_max(float v) {
  v = row16_max(v);
  if constexpr (BS == 32) v = xor_max<16>(v);
  return v;
}
template <int BS>
__device__ __forceinline__ float token_group_sum(float v) {
  v = row16_sum(v);
  if constexpr (BS == 32) v = xor_sum<16>(v);
  return v;
}

// Sum over the VPD lanes that hold the same V dim (adjacent lanes).
template <int VPD>
__device__ __forceinline__ float dim_group_sum(float v) {
  if constexpr (VPD >= 2) v += dpp<0xB1>(v);  // xor 1
  if constexpr (VPD >= 4) v += dpp<0x4E>(v);  // xor 2
  if constexpr (VPD >= 8) v += __shfl_xor(v, 4);
  static_assert(VPD <= 8, "V unit layout");
  return v;
}

#if PA_WAVES_PER_EU_VALU > 0
#define PA_VALU_OCCUPANCY __attribute__((amdgpu_waves_per_eu(PA_WAVES_PER_EU_VALU)))
#else
#define PA_VALU_OCCUPANCY
#endif

// LIST: 0 = one work item per workgroup (grid decomposition); 1 = persistent
// list, one worker per workgroup; 2 = persistent list, one worker per wave;
// 3 = the same as 2 in the slot form (auto without counters).
template <typename QT, typename KVT, int D, int BS, int GP, bool CAP, bool WIN, int LIST = 0>
__global__ void __launch_bounds__(kThreads) PA_VALU_OCCUPANCY pa_partition_valu(const Params p) {
  using T = ValuTraits<QT, KVT>;
  using HM = HeadMap<GP, BS>;
  using PV = typename T::PV;
  constexpr int ESZ = T::kBytes;
  constexpr int X = 16 / ESZ;               // elements per 16-byte chunk / unit
  constexpr int R = 64 / BS;                // lanes per token in the K layout
  constexpr int TILE = D * BS * ESZ;        // bytes of one (block, KV head) K or V tile
  constexpr int NL = TILE / 1024;           // 16-byte loads per lane per tile
  constexpr int VPD = BS * ESZ / 16;        // 16-byte units per V dim row
  constexpr int NF = HM::NF;
  static_assert(NL * 1024 == TILE, "tile must be a multiple of 1 KB");
  static_assert(GP * NL * T::kQW <= 64, "query slice must fit in 64 VGPRs");

  __shared__ float sm_o[kWaves][GP][D];
  __shared__ float sm_m[kWaves][GP];
  __shared__ float sm_l[kWaves][GP];
  __shared__ __attribute__((aligned(16))) PV sm_p[kWaves][2][GP][BS];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok = lane % BS;
  const int r = lane / BS;
  const int tg = lane % VPD;
  int my_head_base = 0;  // first head slot this lane owns after the transpose-reduce
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
    if (rr == r) my_head_base = HM::head_base(rr);

  const char *kcache = reinterpret_cast<const char *>(p.key_cache);
  const char *vcache = reinterpret_cast<const char *>(p.value_cache);
  const size_t blk_stride = (size_t)p.num_kv_heads * TILE;

  // One work item (a partition, a whole v1 sequence, or a piece) with the
  // addressing its tile loads need.
  struct Item {
    Work w;
    const_i32_ptr btab;
    size_t head_off;
  };
  auto make_item = [&](const Work &w) {
    Item it;
    it.w = w;
    it.btab = as_const_table(p.block_tables + (size_t)w.seq * p.max_num_blocks_per_seq);
    it.head_off = (size_t)w.kvh * TILE;
    return it;
  };

  // Query slices of the group's heads for this lane's K chunks, and the
  // ALiBi slope (log2 units) of each head slot this lane owns.
  unsigned qw[GP][NL][T::kQW];
  float slope2[NF];
  auto load_query = [&](const Work &w) {
    const QT *qbase = reinterpret_cast<const QT *>(p.query) +
                      ((size_t)w.seq * p.num_heads + w.head0) * D;
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if (h < w.nh) {
          T::load_q(qbase + h * D + (i * R + r) * X, qw[h][i]);
        } else {
#pragma unroll
          for (int e = 0; e < T::kQW; ++e) qw[h][i][e] = 0u;
        }
      }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int h = my_head_base + j;
      slope2[j] = (p.alibi_slopes && h < w.nh) ? p.alibi_slopes[w.head0 + h] * kLog2e : 0.0f;
    }
  };

  // Online-softmax state of the wave for the current item.
  float m_run[NF], l_run[NF];
  float acc[GP][NL];
  bool poisoned;
  auto reset_state = [&] {
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      m_run[j] = -__builtin_inff();
      l_run[j] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int i = 0; i < NL; ++i) acc[h][i] = 0.0f;
    poisoned = false;
  };

  struct Tile {
    u32x4 k[NL], v[NL];
    bool bad;  // the block-table entry was out of range
  };
  // Out-of-range block-table entries are redirected to block 0 (always
  // addressable) and reported through the tile's bad flag.
  auto load_tile = [&](const Item &it, int blk) {
    Tile t;
    int phys = it.btab[blk];
    t.bad = phys < 0 || phys >= p.num_blocks;
    phys = t.bad ? 0 : phys;
    const char *kb = kcache + (size_t)phys * blk_stride + it.head_off + 16 * lane;
    const char *vb = vcache + (size_t)phys * blk_stride + it.head_off + 16 * lane;
#pragma unroll
    for (int i = 0; i < NL; ++i) t.k[i] = load16_stream(kb + 1024 * i);
#pragma unroll
    for (int i = 0; i < NL; ++i) t.v[i] = load16_stream(vb + 1024 * i);
    return t;
  };

  auto process = [&](const Item &it, int blk, int parity, const Tile &tl) {
    const Work &w = it.w;
    poisoned |= tl.bad;
    // Logits: partial dots over this lane's chunks, then transpose-reduce.
    float s[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < NL; ++i) a = T::qk(a, qw[h][i], tl.k[i]);
      s[h] = a;
    }
    transpose_reduce<GP, BS>(s);
    const int t_abs = blk * BS + tok;
    float alpha[NF], pj[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      float x = scaled_logit<CAP, std::is_same<QT, float>::value>(p, s[j]) +
                slope2[j] * (float)(t_abs - w.t_ref);
      x = in_span<WIN>(t_abs, w.t_lo, w.span) ? x : -__builtin_inff();
      const float bm = token_group_max<BS>(x);
      const float m_new = fmaxf(m_run[j], bm);
      alpha[j] = (m_new == -__builtin_inff()) ? 1.0f : fast_exp2(m_run[j] - m_new);
      pj[j] = fast_exp2(x - m_new);
      l_run[j] = l_run[j] * alpha[j] + pj[j];
      m_run[j] = m_new;
    }
    // P into the V layout through LDS.
#pragma unroll
    for (int j = 0; j < NF; ++j) sm_p[wv][parity][my_head_base + j][tok] = (PV)pj[j];
    wave_lds_sync();
    // Rescale factor of every head, from the lanes that own it.
    float a_bc[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h)
      a_bc[h] = readlane(alpha[h - HM::head_base(HM::src_group(h))], HM::src_group(h) * BS);
    const int vlo = w.t_lo - blk * BS;  // window start relative to the block
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      unsigned vw[T::kPW];
      T::v_words(tl.v[i], vw);
      T::template mask_v<WIN>(vw, tg * X, vlo, w.span);
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float a_h = a_bc[h];
        const unsigned *pp = reinterpret_cast<const unsigned *>(&sm_p[wv][parity][h][tg * X]);
        unsigned pw[T::kPW];
#pragma unroll
        for (int e = 0; e < T::kPW; ++e) pw[e] = pp[e];
        acc[h][i] = T::pv(acc[h][i] * a_h, pw, vw);
      }
    }
  };

  // The wave's blocks of the item (blk_begin + first, then every stride-th;
  // stride 4 when the workgroup shares the item, 1 for a list worker): two
  // tiles ping-pong, and while block blk is consumed the loads of the wave's
  // next block are in flight.  The loop runs whole pairs with no exit
  // between them and always issues its loads, so the wait before a block
  // covers only that block's tile; the scheduling barriers keep each
  // prefetch ahead of the block's compute.  On entry ta holds (or is
  // loading) the wave's first block.
  auto run_steps = [&](const Item &it, Tile &ta, Tile &tb, int first, auto stride_c) {
    constexpr int S = decltype(stride_c)::value;
    const Work &w = it.w;
    auto parity = [&](int b) { return ((b - w.blk_begin) / S) & 1; };
    int blk = w.blk_begin + first;
    int left = blk < w.blk_end ? (w.blk_end - blk + S - 1) / S : 0;
    while (left >= 3) {
      tb = load_tile(it, blk + S);
      __builtin_amdgcn_sched_barrier(0);
      process(it, blk, parity(blk), ta);
      ta = load_tile(it, blk + 2 * S);
      __builtin_amdgcn_sched_barrier(0);
      process(it, blk + S, parity(blk + S), tb);
      blk += 2 * S;
      left -= 2;
    }
    if (left == 2) {
      tb = load_tile(it, blk + S);
      __builtin_amdgcn_sched_barrier(0);
      process(it, blk, parity(blk), ta);
      process(it, blk + S, parity(blk + S), tb);
    } else if (left == 1) {
      process(it, blk, parity(blk), ta);
    }
  };
  // The wave's first tile of an item, if it has a block.
  auto first_tile = [&](const Item &it, Tile &ta, int first) {
    const int b0 = it.w.blk_begin + first;
    if (b0 < it.w.blk_end) ta = load_tile(it, b0);
  };

  // Wave totals per head, then the cross-wave merge and the stores.  Lane
  // indices are re-read here (epi_tid) rather than carried across the list
  // form's item loop.
  auto finish_item = [&](const Item &it) {
    const int et = epi_tid(), el = et & 63, ew = et >> 6, etg = el % VPD;
#pragma unroll
    for (int j = 0; j < NF; ++j) l_run[j] = token_group_sum<BS>(l_run[j]);
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const int g = HM::src_group(h);
      const int j = h - HM::head_base(g);
      const float mh = readlane(m_run[j], g * BS);
      const float lh = readlane(l_run[j], g * BS);
      if (el == 0) {
        sm_m[ew][h] = mh;
        sm_l[ew][h] = poisoned ? __builtin_nanf("") : lh;
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float v = dim_group_sum<VPD>(acc[h][i]);
        if (etg == 0) sm_o[ew][h][(64 * i + el) / VPD] = v;
      }
    }
    __syncthreads();
    finish_partition<QT, D, GP, D>(p, it.w, sm_o, sm_m, sm_l);
  };

  // A list worker's epilogue, from registers: every head's running max and
  // sum come from the lanes that own it; lane l with l % VPD == 0 holds dim
  // (64 i + l) / VPD of each head.
  auto finish_wave = [&](const Item &it) {
    const Work &w = it.w;
    const int el = epi_tid() & 63, etg = el % VPD;
#pragma unroll
    for (int j = 0; j < NF; ++j) l_run[j] = token_group_sum<BS>(l_run[j]);
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const int g = HM::src_group(h);
      const int j = h - HM::head_base(g);
      const float mh = readlane(m_run[j], g * BS);
      const float lh = readlane(l_run[j], g * BS);
      const float lsum = poisoned ? __builtin_nanf("") : lh;
      const float scale = p.v_scale / lh;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float v = dim_group_sum<VPD>(acc[h][i]);
        if (h < w.nh && etg == 0)
          piece_elem<QT, D>(p, w, h, (64 * i + el) / VPD,
                            lsum != lsum ? __builtin_nanf("") : v * scale);
      }
      if (h < w.nh && w.v2 && el == 0) piece_stats(p, w, h, mh, lsum);
    }
    if (w.v2) {
      if constexpr (LIST == 3) piece_slot_padding(p, w, el);  // the reduce kernel merges
      else if (p.tmp_f32) piece_arrive<QT, float, D>(p, w);
      else piece_arrive<QT, QT, D>(p, w);
    }
  };

  if constexpr (LIST == 2 || LIST == 3) {
    // Persistent, one worker per wave: every wave walks the pieces of its
    // share of the work list in order, on its own (many small items: a
    // wave's epilogue then overlaps the other waves' streaming).  The next
    // piece's query and first tile are requested before this piece's
    // epilogue, which then overlaps their latency.  LIST 3: the slot form
    // (pieces to partition slots for the reduce kernel, no arrivals).
    ListCursor cur;
    if (!list_begin(p, cur, (int)blockIdx.x * kWaves + wv, (int)gridDim.x * kWaves)) return;
    Work w;
    if (!list_next<QT, D, LIST == 3>(p, BS, GP, cur, w)) return;
    Item it = make_item(w);
    load_query(w);
    Tile ta, tb;
    first_tile(it, ta, 0);
    while (true) {
      reset_state();
      run_steps(it, ta, tb, 0, std::integral_constant<int, 1>{});
      Work wn;
      const bool more = list_next<QT, D, LIST == 3>(p, BS, GP, cur, wn);
      Item itn;
      if (more) {
        itn = make_item(wn);
        load_query(wn);
        first_tile(itn, ta, 0);
      }
      finish_wave(it);
      if (!more) break;
      it = itn;
    }
  } else if constexpr (LIST == 1) {
    // Persistent, one worker per workgroup (few, large items: the four
    // waves share each piece and merge through LDS).  Prefetch as above;
    // the barrier frees the LDS of one piece's epilogue for the next.
    ListCursor cur;
    if (!list_begin(p, cur, (int)blockIdx.x, (int)gridDim.x)) return;
    Work w;
    if (!list_next<QT, D>(p, BS, GP, cur, w)) return;
    Item it = make_item(w);
    load_query(w);
    Tile ta, tb;
    first_tile(it, ta, wv);
    while (true) {
      reset_state();
      run_steps(it, ta, tb, wv, std::integral_constant<int, kWaves>{});
      Work wn;
      const bool more = list_next<QT, D>(p, BS, GP, cur, wn);
      Item itn;
      if (more) {
        itn = make_item(wn);
        load_query(wn);
        first_tile(itn, ta, wv);
      }
      finish_item(it);
      __syncthreads();
      if (!more) break;
      it = itn;
    }
  } else {
    Work w;
    if (!begin_work<QT, D>(p, BS, GP, w)) return;
    const Item it = make_item(w);
    load_query(w);
    reset_state();
    Tile ta, tb;
    first_tile(it, ta, wv);
    run_steps(it, ta, tb, wv, std::integral_constant<int, kWaves>{});
    finish_item(it);
  }
}

}  // namespace pa
