// Partition-phase kernel, MFMA form: for GQA groups wide enough (5..16 query
// heads per KV head) that QK^T and PV become real dense 16-row tiles.
//
// A wave consumes 32 tokens per step (two 16-token blocks, or one 32-token
// block).
//   S^T = K . Q^T with v_mfma_f32_16x16x32 (bf16/f16), one per 16-token
//        sub-tile and 32-dim k-step: A = 16 tokens x 32 dims of K, B = 32 dims
//        x 16 query heads (the group, zero padded).  Lane l feeds token l%16
//        with the 16-byte K chunk 4i + l/16 of load i: the coalesced 1 KB per
//        instruction read of the [D/x][bs][x] layout (fp8 chunks hold 16 dims
//        and feed two k-steps; the query slices follow the same dim order).
//   O^T += V^T . P^T with v_mfma_f32_16x16x32: lane (n, g) = (l%16, l/16)
//        feeds head-dim row 16t + n with 8 consecutive tokens, i.e. one
//        16-byte load of the [D][bs] V layout (8 bytes for fp8).  The S^T
//        accumulators leave lane (n, g) with tokens 4g..4g+3 of each 16-token
//        sub-tile; two permlane swaps (32 then 16) regroup the packed P so
//        that lane group g holds tokens 8(g^1) .. 8(g^1)+7, the same tokens
//        its V row covers: P never goes through LDS.
// Each lane keeps the running max / sum of one query head (l%16), so the
// online-softmax rescale of O needs no broadcast.  fp8 E4M3FN keys are
// widened exactly to the query's 16-bit type, values to fp16 (P in fp16).
//
// ROWS: the [num_blocks, Hkv, block_size, head_size] layout (16-bit only).
// K and V rows are both loaded as whole 1 KB runs of consecutive tokens and
// pass through a per-wave LDS slab.  K rows are read back as the same QK
// operands (lane (n, g), k-step ks: the 16 bytes of dims 32 ks + 8 g of
// token n), with a row stride that spreads the 16 rows of one read over all
// banks.  V rows are read back column-wise with the gfx950 transposing LDS
// read
// (ds_read_b64_tr_b16): within each 16-lane group, lane 4 j + q names 4
// consecutive values of one row and lane i receives value i % 4 of the
// rows named by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4 -- so lanes
// naming (row t0 + j, dims d0 + 4 q ..) hand lane n the values of dim d0 + n
// at tokens t0 .. t0 + 3: half a V^T operand per read.
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
__device__ __forceinline__ f32x4 mfma_pv(const u32x4 &a, const u32x4 &b, const f32x4 &c,
                                         __bf16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_pv(const u32x4 &a, const u32x4 &b, const f32x4 &c,
                                         _Float16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Zero the 16-bit elements of tokens outside [lo, lo + span) in an 8-token V
// operand whose first element is token 0.
template <bool WIN>
__device__ __forceinline__ u32x4 mask_v8(u32x4 v, int lo, int span) {
  return u32x4{v.x & keep_pair_mask<WIN>(0, lo, span), v.y & keep_pair_mask<WIN>(2, lo, span),
               v.z & keep_pair_mask<WIN>(4, lo, span), v.w & keep_pair_mask<WIN>(6, lo, span)};
}

// Regroups packed P (two 4-token pieces per lane: p0 from sub-tile 0, p1
// from sub-tile 1, tokens 4g..4g+3 each) so that lane group g holds the 8
// tokens 8(g^1) .. 8(g^1)+7 of the 32-token step, in order.
__device__ __forceinline__ u32x4 regroup_p(const u32x2 &p0, const u32x2 &p1) {
  // Step 1 (lanes l <-> l^32): lower half gets P0 of groups g and g+2, upper
  // half P1 of groups g-2 and g.
  auto a0 = __builtin_amdgcn_permlane32_swap(p0.x, p1.x, false, false);
  auto a1 = __builtin_amdgcn_permlane32_swap(p0.y, p1.y, false, false);
  // Step 2 (rows 2k <-> 2k+1): even rows keep their second value and take
  // the odd row's second value; odd rows take the even row's first value.
  auto b0 = __builtin_amdgcn_permlane16_swap(a0[1], a0[0], false, false);
  auto b1 = __builtin_amdgcn_permlane16_swap(a1[1], a1[0], false, false);
  return u32x4{b0[0], b1[0], b0[1], b1[1]};
}

// Waves per SIMD the register allocator must leave room for: two, with
// both ping-pong tiles in registers.  (fp8 tiles are half the size, but three
// waves make the allocator spill and measured slower than two.)
// The persistent list form runs one workgroup per CU, one wave per SIMD:
// the whole register file is its own.
template <typename KVT, bool LIST>
constexpr int mfma_waves_per_eu() {
  if constexpr (LIST) return 1;
  else if constexpr (PA_WAVES_PER_EU_MFMA > 0) return PA_WAVES_PER_EU_MFMA;
  else return 2;
}

// Barrier over LDS only: orders the workgroup's LDS traffic without waiting
// for its global stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Transposing LDS read of four 16-bit values (lane layout above).
__device__ __forceinline__ u32x2 lds_read_tr16(const char *lds_ptr) {
  typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 h4;
  typedef __attribute__((address_space(3))) h4 lds_h4;
  const h4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (lds_h4 *)((__attribute__((address_space(3))) char *)lds_ptr));
  return __builtin_bit_cast(u32x2, v);
}

template <typename QT, typename KVT, int D, int BS, bool CAP, bool WIN, bool ROWS = false,
          bool LIST = false>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(mfma_waves_per_eu<KVT, LIST>())))
    pa_partition_mfma(const Params p) {
  constexpr bool kFp8 = std::is_same<KVT, fp8e4m3>::value;
  using PT = typename std::conditional<kFp8, _Float16, KVT>::type;  // P.V operand type
  static_assert(kFp8 || std::is_same<KVT, QT>::value, "16-bit cache must match the query type");
  constexpr int ESZ = kFp8 ? 1 : 2;
  constexpr int TILE = D * BS * ESZ;          // bytes of one K or V tile
  constexpr int BPS = 32 / BS;                // blocks per 32-token step
  constexpr int NLK = D * 16 * ESZ / 1024;    // 16-byte K loads per lane per 16-token sub-tile
  constexpr int NKS = D / 32;                 // 32-dim k-steps of QK
  constexpr int NDT = D / 16;                 // 16-dim tiles of the output
  constexpr int OSTR = D + 4;                 // padded LDS row (bank spread)
  static_assert(NLK >= 1 && NLK * (kFp8 ? 2 : 1) == NKS, "K sub-tile geometry");
  static_assert(!ROWS || !kFp8, "the block-rows layout has 16-bit caches only");
  // ROWS: V slab rows (one per step token, 32 bytes of padding spread the
  // four rows a transposing read touches over distinct banks), K slab rows
  // (16 bytes of padding: the 16 token rows of a K operand read start on
  // distinct 4-bank groups), tokens per 1 KB load, lanes per token row.
  constexpr int VSTR = 2 * D + 32;
  constexpr int KSTR = 2 * D + 16;
  constexpr int VTPL = 512 / D;
  constexpr int VR = D / 8;

  __shared__ float sm_o[kWaves][16][OSTR];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ __attribute__((aligned(16))) char sm_v[ROWS ? kWaves * 32 * VSTR : 16];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;   // query head of the group (MFMA column) / V dim row
  const int g = lane >> 4;   // lane group: k-slot block / row block
  const int vtok = 8 * (g ^ 1);  // first of the 8 step tokens this lane's P / V operands hold

  const char *kcache = reinterpret_cast<const char *>(p.key_cache);
  const char *vcache = reinterpret_cast<const char *>(p.value_cache);
  const size_t blk_stride = (size_t)p.num_kv_heads * TILE;

  // One work item (a partition, or a whole v1 sequence, of one (sequence, KV
  // head)) with the addressing its tile loads need.
  struct Item {
    Work w;
    const_i32_ptr btab;
    size_t head_off;
    int tok_begin, n_steps;
  };
  auto make_item = [&](const Work &w) {
    Item it;
    it.w = w;
    it.btab = as_const_table(p.block_tables + (size_t)w.seq * p.max_num_blocks_per_seq);
    it.head_off = (size_t)w.kvh * TILE;
    it.tok_begin = w.blk_begin * BS;
    it.n_steps = ((w.blk_end - w.blk_begin) * BS + 31) / 32;
    return it;
  };

  // B operands of QK: 8 query values per lane and k-step, in the dim order
  // of the K chunks (16-bit: dims 32ks + 8g + e; fp8: chunk 4i + g of 16 dims,
  // halves ks = 2i and 2i + 1).
  u32x4 qop[NKS];
  float slope2 = 0.0f;
  auto load_query = [&](const Work &w) {
    const QT *q = reinterpret_cast<const QT *>(p.query) +
                  ((size_t)w.seq * p.num_heads + w.head0 + n) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int dim0 = kFp8 ? (16 * (4 * (ks / 2) + g) + 8 * (ks % 2)) : (32 * ks + 8 * g);
      qop[ks] = (n < w.nh) ? load16(q + dim0) : u32x4{0u, 0u, 0u, 0u};
    }
    slope2 = (p.alibi_slopes && n < w.nh) ? p.alibi_slopes[w.head0 + n] * kLog2e : 0.0f;
  };

  // Online-softmax state of the wave for the current item.
  float m_run, l_run;
  f32x4 oacc[NDT];
  bool poisoned;
  auto reset_state = [&] {
    m_run = -__builtin_inff();
    l_run = 0.0f;
#pragma unroll
    for (int t = 0; t < NDT; ++t) oacc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    poisoned = false;
  };

  // K: sub-tile h, load i -> chunk 4i + g, token 16h + n of the step.
  // V: dim tile t -> dim 16t + n, tokens vtok .. vtok + 7 of the step.
  // bad: a block-table entry of the step was out of range.
  using VOp = typename std::conditional<kFp8, u32x2, u32x4>::type;
  struct Tile {
    u32x4 k[2][NLK];
    VOp v[NDT];
    bool bad;
  };

  // Out-of-range block-table entries are redirected to block 0 (always
  // addressable) and reported through the tile's bad flag; the second block
  // of a step past the range end is read from block 0 too, and all its tokens
  // are masked.
  // The V operand's block differs between lane groups when two blocks make
  // a step; it is selected as an index and addressed from the cache base, so
  // the loads stay global (a per-lane select between two pointers compiles to
  // flat loads, whose completion order forces full waits on every step).
  auto load_tile = [&](const Item &it, int step) {
    Tile tl;
    tl.bad = false;
    int phys[BPS];
    const char *kb[BPS];
#pragma unroll
    for (int b = 0; b < BPS; ++b) {
      const int lb = it.w.blk_begin + step * BPS + b;
      phys[b] = 0;
      if (lb < it.w.blk_end) {
        phys[b] = it.btab[lb];
        if (phys[b] < 0 || phys[b] >= p.num_blocks) {
          tl.bad = true;
          phys[b] = 0;
        }
      }
      kb[b] = kcache + (size_t)phys[b] * blk_stride + it.head_off;
    }
    if constexpr (ROWS) {
      // K and V load i: tokens VTPL i .. VTPL i + VTPL - 1 (one block), 1 KB
      // each; the K loads fill tl.k in order (2 NLK == NDT of them).
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const int tok = VTPL * i + lane / VR;
        const size_t row = (size_t)phys[(VTPL * i) / BS] * blk_stride + it.head_off +
                           (tok % BS) * (2 * D) + 16 * (lane % VR);
        tl.k[i / NLK][i % NLK] = load16_stream(kcache + row);
        tl.v[i] = load16_stream(vcache + row);
      }
      return tl;
    }
    const int vphys = (BPS == 1 || vtok < BS) ? phys[0] : phys[BPS - 1];
    const char *vb = vcache + (size_t)vphys * blk_stride + it.head_off;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < NLK; ++i) {
        const int tok = 16 * h + n;
        tl.k[h][i] = load16_stream(kb[tok / BS] + (4 * i + g) * (BS * 16) + (tok % BS) * 16);
      }
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      const char *src = vb + ((16 * t + n) * BS + vtok % BS) * ESZ;
      if constexpr (kFp8) tl.v[t] = load8_stream(src);
      else tl.v[t] = load16_stream(src);
    }
    return tl;
  };

  char *const vslab = sm_v + (ROWS ? wv * 32 * VSTR : 0);
  auto process = [&](const Item &it, int step, const Tile &tl) {
    poisoned |= tl.bad;
    // ROWS: V rows into the wave's slab, then the transposed operands out
    // (the wave's LDS accesses execute in order; the previous step's reads
    // were consumed by its PV products before these writes).
    u32x4 vrows[ROWS ? NDT : 1];
    u32x4 krows[2][NLK];
    if constexpr (ROWS) {
      // K rows in, the QK operands out; then the V rows over them (the
      // wave's LDS accesses execute in order).
#pragma unroll
      for (int i = 0; i < NDT; ++i)
        *reinterpret_cast<u32x4 *>(vslab + (VTPL * i + lane / VR) * KSTR + 16 * (lane % VR)) =
            tl.k[i / NLK][i % NLK];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < NLK; ++i)
          krows[h][i] =
              *reinterpret_cast<const u32x4 *>(vslab + (16 * h + n) * KSTR + 64 * i + 16 * g);
#pragma unroll
      for (int i = 0; i < NDT; ++i)
        *reinterpret_cast<u32x4 *>(vslab + (VTPL * i + lane / VR) * VSTR + 16 * (lane % VR)) =
            tl.v[i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      const char *rd = vslab + (vtok + (n >> 2)) * VSTR + 8 * (n & 3);
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const u32x2 lo = lds_read_tr16(rd + 32 * t);
        const u32x2 hi = lds_read_tr16(rd + 4 * VSTR + 32 * t);
        vrows[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    }
    // S^T for each 16-token sub-tile: lane holds head n, tokens 16h + 4g + e.
    f32x4 st[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < NLK; ++i) {
        if constexpr (kFp8) {
          const u32x4 kw = tl.k[h][i];
          const u32x4 lo = {fp8x2_to<false>(kw.x, QT()), fp8x2_to<true>(kw.x, QT()),
                            fp8x2_to<false>(kw.y, QT()), fp8x2_to<true>(kw.y, QT())};
          const u32x4 hi = {fp8x2_to<false>(kw.z, QT()), fp8x2_to<true>(kw.z, QT()),
                            fp8x2_to<false>(kw.w, QT()), fp8x2_to<true>(kw.w, QT())};
          c = mfma_qk(lo, qop[2 * i], c, QT());
          c = mfma_qk(hi, qop[2 * i + 1], c, QT());
        } else if constexpr (ROWS) {
          c = mfma_qk(krows[h][i], qop[i], c, QT());
        } else {
          c = mfma_qk(tl.k[h][i], qop[i], c, QT());
        }
      }
      st[h] = c;
    }
    // Scale (and soft cap), ALiBi, window / tail mask, step max over the
    // head's tokens.
    const int t0 = it.tok_begin + 32 * step;
    float x[2][4];
    float bm = -__builtin_inff();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 16 * h + 4 * g + e;
        float v = scaled_logit<CAP>(p, st[h][e]) + slope2 * (float)(t - it.w.t_ref);
        v = in_span<WIN>(t, it.w.t_lo, it.w.span) ? v : -__builtin_inff();
        x[h][e] = v;
        bm = fmaxf(bm, v);
      }
    bm = xor_max<32>(xor_max<16>(bm));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = (m_new == -__builtin_inff()) ? 1.0f : fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.0f;
    u32x2 pk[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = fast_exp2(x[h][e] - m_new);
        psum += pe[e];
      }
      pk[h] = u32x2{pack2(pe[0], pe[1], PT()), pack2(pe[2], pe[3], PT())};
    }
    l_run = l_run * alpha + psum;
    const u32x4 pop = regroup_p(pk[0], pk[1]);
    const int vlo = it.w.t_lo - (t0 + vtok);  // window start relative to this lane's V operand
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      u32x4 va;
      if constexpr (kFp8) {
        va = u32x4{fp8x2_to<false>(tl.v[t].x, _Float16()), fp8x2_to<true>(tl.v[t].x, _Float16()),
                   fp8x2_to<false>(tl.v[t].y, _Float16()), fp8x2_to<true>(tl.v[t].y, _Float16())};
      } else if constexpr (ROWS) {
        va = vrows[t];
      } else {
        va = tl.v[t];
      }
      va = mask_v8<WIN>(va, vlo, it.w.span);
      oacc[t] = mfma_pv(va, pop, oacc[t] * alpha, PT());
    }
  };

  // The wave's steps of the item (first, first + stride, ...; stride 4 when
  // the workgroup shares the item, 1 for a list worker): two tiles
  // ping-pong, and while step st is consumed the loads of the wave's next
  // step are in flight.  The loop runs whole pairs and has no exit between them, and
  // every load in it is always issued, so the wait before a step covers only
  // that step's tile (a mid-pair exit would merge a path with the other tile
  // still in flight into the back edge).  The scheduling barriers keep each
  // prefetch ahead of the step's compute.  On entry ta is loading the wave's
  // first step.
  // on_second() runs once, after the wave's second step: the first tile
  // the wave waited for that was requested inside this call.
  auto run_steps = [&](const Item &it, Tile &ta, Tile &tb, int first, auto stride_c,
                       auto on_second) {
    constexpr int S = decltype(stride_c)::value;
    int st = first;
    int left = st < it.n_steps ? (it.n_steps - st + S - 1) / S : 0;
    bool hook = true;
    while (left >= 3) {
      tb = load_tile(it, st + S);
      __builtin_amdgcn_sched_barrier(0);
      process(it, st, ta);
      ta = load_tile(it, st + 2 * S);
      __builtin_amdgcn_sched_barrier(0);
      process(it, st + S, tb);
      if (hook) {
        on_second();
        hook = false;
      }
      st += 2 * S;
      left -= 2;
    }
    if (left == 2) {
      tb = load_tile(it, st + S);
      __builtin_amdgcn_sched_barrier(0);
      process(it, st, ta);
      process(it, st + S, tb);
      if (hook) on_second();
    } else if (left == 1) {
      process(it, st, ta);
    }
  };
  auto no_hook = [] {};

  // The waves' states into LDS (wave totals: the four lanes of head n hold
  // partial sums over their tokens), then an LDS barrier.
  auto stage_item = [&] {
    const float l_tot = xor_sum<32>(xor_sum<16>(l_run));
    // Lane indices re-read here (see epi_tid) rather than carried in
    // registers across the list form's item loop.
    const int et = epi_tid(), ew = et >> 6, en = et & 15, eg = (et & 63) >> 4;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) sm_o[ew][en][16 * t + 4 * eg + e] = oacc[t][e];
    if (eg == 0) {
      sm_m[ew][en] = m_run;
      sm_l[ew][en] = poisoned ? __builtin_nanf("") : l_tot;
    }
    lds_barrier();
  };
  // Cross-wave merge and stores of one item.
  auto finish_item = [&](const Item &it) {
    stage_item();
    finish_partition<QT, D, 16, OSTR>(p, it.w, sm_o, sm_m, sm_l);
  };

  if constexpr (LIST) {
    // Persistent, one worker per workgroup: the pieces of its share of the
    // work list in order.  The next piece is found while this one streams;
    // its query and first tile are requested before this piece's epilogue
    // (cross-wave merge, stores, arrivals), which then overlaps their
    // latency; the barrier frees the LDS of one piece's epilogue for the
    // next.  (The GQA groups this kernel serves make few, large items per
    // worker, where one worker per wave would cut every item into many
    // pieces.)
    ListCursor cur;
    if (!list_begin(p, cur, (int)blockIdx.x, (int)gridDim.x)) return;
    Work w;
    if (!list_next<QT, D>(p, BS, 16, cur, w)) return;
    Item it = make_item(w);
    load_query(w);
    Tile ta, tb;
    if (wv < it.n_steps) ta = load_tile(it, wv);
    ListPend pend{};
    int pend_old = 0;
    while (true) {
      Work wn;
      const bool more = list_next<QT, D>(p, BS, 16, cur, wn);
      const bool final_cut = !more && it.w.v2;
      int early = 0;
      if (final_cut && threadIdx.x == 0)
        early = (int)coherent_load(item_counter(p, it.w.seq, it.w.xslot));
      reset_state();
      run_steps(it, ta, tb, wv, std::integral_constant<int, kWaves>{},
                [&] { list_pend_arrive(p, pend, pend_old); });
      // Nothing is in flight after the wave's last step; this makes its
      // earlier partial stores performed for the arrivals.
      __builtin_amdgcn_s_waitcnt(0x0F70);
      Item itn;
      if (more) {
        itn = make_item(wn);
        load_query(wn);
        if (wv < itn.n_steps) ta = load_tile(itn, wv);
      }
      stage_item();
      finish_list_piece<QT, D, 16, OSTR>(p, it.w, sm_o, sm_m, sm_l, pend, final_cut, early,
                                         pend_old);
      __syncthreads();
      if (!more) break;
      it = itn;
    }
  } else {
    Work w;
    if (!begin_work<QT, D>(p, BS, 16, w)) return;
    const Item it = make_item(w);
    load_query(w);
    reset_state();
    Tile ta, tb;
    if (wv < it.n_steps) ta = load_tile(it, wv);
    run_steps(it, ta, tb, wv, std::integral_constant<int, kWaves>{}, no_hook);
    finish_item(it);
  }
}

}  // namespace pa
