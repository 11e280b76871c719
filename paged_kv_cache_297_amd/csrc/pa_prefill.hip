// Paged prefill attention (page "Layer 3: Attention prefill/decode dispatch",
// dispatch_prefill: flash attention over variable-length sequences whose keys
// and values are read through block tables from a [num_blocks, Hkv, bs, D]
// cache, with cumulative query / key offsets, a causal flag, a left / right
// window and a logit soft cap).  The queries of a sequence are its last nq
// positions: query token i sits at position nk - nq + i.
//
// A workgroup owns 64 or 128 query columns -- (query token, query head) pairs
// of one KV head, one or two 16-column MFMA tiles per wave -- and walks the
// keys its columns can see in steps of 32.  Each step's K and V tiles go
// from the cache straight into LDS with direct-to-LDS loads, through a ring
// of three stages (one barrier per step), and feed every wave's column
// tiles.  Per wave, column tile and step, with v_mfma_f32_16x16x32:
//   S^T = K . Q^T   (A = 16 keys x 32 dims of K, B = 32 dims x 16 columns of
//                    Q held in registers), two 16-key sub-tiles;
//   masks, soft cap, online softmax per column (max / sum across the four
//   lanes of a column);
//   O^T += V^T . P^T (A = 16 dims x 8 keys of V read with the transposing LDS
//                    read, B = P as the QK product left it in the lanes).
#include "pa_launch_kernel.h"
#include "pa_partition_mfma.h"
#include "pa_prefill.h"

namespace pa {

// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin in
// launch order.  With PA_PREFILL_XCD_MAP the launch index is remapped so that
// each XCD owns a fixed set of (sequence, KV head) pairs, whose query tiles
// read the same keys and values and then share one L2.  It runs them in one
// of two orders (p.tile_major, set by the host):
//   - pair-major: one pair's tiles (heaviest first), then the next pair's,
//     so that few pairs' keys and values are in flight at once -- for
//     batches whose tiles cost about the same (chunked prefill: every tile
//     sees the whole prefix);
//   - tile-major: the heaviest tiles of all its pairs first -- for causal
//     batches whose tiles' costs differ widely (a fresh prompt's tile t sees
//     t + 1 steps), where pair-major leaves the last pair's longest tiles
//     for the end: a list-scheduling model of 8 pairs x 64 such tiles on 96
//     slots gives 14% over the ideal makespan pair-major, 2.4% tile-major
//     (measured on MI355X: 8 fresh 2048-token prompts 0.333 -> 0.317 ms; the
//     chunked batch, tile-major, 1.05 -> 1.19 ms from L2 misses).
// With a pair count not divisible by 8, tile-major ignores the XCDs.
#ifndef PA_PREFILL_XCD_MAP
#define PA_PREFILL_XCD_MAP 1
#endif
constexpr int kXcds = 8;

// (bx, by, bz) = (tile rank from the heaviest, KV head, sequence).
__device__ __forceinline__ void prefill_item(const PrefillParams &p, int &bx, int &by, int &bz) {
  bx = blockIdx.x;
  by = blockIdx.y;
  bz = blockIdx.z;
#if PA_PREFILL_XCD_MAP
  const unsigned long long gx = gridDim.x, gy = gridDim.y;
  const unsigned long long pairs = gy * gridDim.z;
  const unsigned long long total = gx * pairs;
  const unsigned long long lin = bx + gx * (by + gy * bz);
  if (p.tile_major) {
    unsigned long long rank, pair;
    if (pairs % kXcds == 0) {
      // Launch lin = 8 s + k runs on XCD k as its s-th workgroup.
      const unsigned long long per = pairs / kXcds, k = lin % kXcds, s = lin / kXcds;
      rank = s / per;
      pair = k * per + s % per;
    } else {
      rank = lin / pairs;
      pair = lin % pairs;
    }
    bx = (int)rank;
    by = (int)(pair % gy);
    bz = (int)(pair / gy);
  } else {
    // A bijection on [0, whole): launch lin = 8 s + k (XCD k, round s) runs
    // item k * whole / 8 + s in (tile, KV head, sequence) order.
    const unsigned long long whole = total - total % kXcds;  // the rest keep their place
    if (lin < whole) {
      const unsigned long long item = (lin % kXcds) * (whole / kXcds) + lin / kXcds;
      bx = (int)(item % gx);
      by = (int)((item / gx) % gy);
      bz = (int)(item / (gx * gy));
    }
  }
#endif
}

// Sum of the two 16-bit values of a packed word, added to c in fp32.
__device__ __forceinline__ float dot2_sum(unsigned w, float c, __bf16) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), c, false);
}
__device__ __forceinline__ float dot2_sum(unsigned w, float c, _Float16) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                __builtin_bit_cast(f16x2, 0x3c003c00u), c, false);
}

// Lazy rescaling of the running softmax state: a column keeps its reference
// max until the running max rises by more than this (log2 units), so its
// weights exp2(s - m_ref) stay at most 2^8 (exact in the 16-bit P operands
// and far from overflow in the fp32 sums), and the accumulators are rescaled
// only on those rare steps instead of on nearly every one.  The output, the
// weighted sum over the sum of weights, is the same in exact arithmetic for
// any reference.
constexpr float kLazyRescale = 8.0f;


// Waves per SIMD the register allocator must leave room for: three at head
// size 128 (three 51 KB rings fill a CU's LDS), four at 64.
template <int D>
constexpr int prefill_waves_per_eu() {
  return D == 64 ? 4 : 3;
}

// Geometry of the ring: K and V tiles loaded by direct-to-LDS loads
// (global_load_lds_dwordx4: lane l of a wave writes its 16 bytes at
// M0 + 16 l), three stages deep.  One load moves 1 KB, KPI whole key rows;
// lane l fetches chunk l / KPI (8 dims) of key l % KPI, so within the load
// the 16-byte chunks are stored chunk-major: (key j, chunk c) at
// 16 (KPI c + j).  Loads sit IB = 1 KB + PAD apart.  With that layout
//   - a QK operand read (16 lanes: keys n = 0..15, one chunk) touches 16
//     distinct 16-byte bank groups (the pad shifts successive loads by a
//     quarter or half of the banks), and
//   - a transposing read of V (16 lanes: four keys x four 4-dim pieces)
//     touches 16 distinct 8-byte bank pairs,
// and both have per-lane bases with compile-time offsets for the k-step,
// the 16-key sub-tile, the 16-dim output tile and the 4-key half.
template <int D>
struct PrefillRing {
  static constexpr int ROWB = D * 2;                    // bytes of one key row
  static constexpr int KPI = 1024 / ROWB;               // keys per load (4 or 8)
  static constexpr int PAD = D == 128 ? 64 : 128;
  static constexpr int IB = 1024 + PAD;                 // LDS bytes per load
  static constexpr int NI = kPrefillStep / KPI;         // loads per tile and step
  static constexpr int IPW = NI / kWaves;               // ... per wave
  static constexpr int TILE = NI * IB;                  // one K (or V) tile
  static constexpr int STAGE = 2 * TILE;                // K tile, then V tile
  static constexpr int NSTAGE = 3;
  static constexpr int BYTES = NSTAGE * STAGE;
  static_assert(IPW >= 1 && IPW * kWaves == NI, "whole loads per wave");
  static_assert(KPI == 4 || KPI == 8, "16-bit rows of 64 or 128 dims");
};

// s_waitcnt immediate that waits until at most n vector memory operations
// of the wave are outstanding (LDS and export counts left alone).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Address of a __shared__ object in the LDS aperture.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) char *)p;
}

// One direct-to-LDS load: 16 bytes from each lane's address to LDS address
// lds + 16 * lane (lds uniform; M0 must hold it one wait state before the
// load).  Issued from asm so that the compiler does not track it: given LDS
// addresses that differ only at run time (the ring stage), it would
// otherwise wait for every load in flight before each LDS read, the
// prefetched stages included.  The load has no result register; the ring's
// own s_waitcnt vmcnt waits order every read of its data.
__device__ __forceinline__ void lds_dma16(const void *src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}

template <typename QT, int D, int BS, int NT, bool CAP>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(prefill_waves_per_eu<D>())))
    pa_prefill_kernel(const PrefillParams p) {
  // NT: 16-column MFMA tiles per wave
  constexpr int NKS = D / 32;                  // 32-dim k-steps of QK^T
  constexpr int NDT = D / 16;                  // 16-dim output tiles
  constexpr int NSUB = kPrefillStep / 16;      // 16-key sub-tiles per step
  constexpr int NHALF = kPrefillStep / 32;     // 32-key P.V slices per step
  static_assert(kPrefillStep % BS == 0, "a step covers whole blocks");

  using RG = PrefillRing<D>;
  __shared__ __attribute__((aligned(1024))) char ring[RG::BYTES];
  __shared__ int sm_bad;

  int bx, by, bz;
  prefill_item(p, bx, by, bz);
  const int tile = p.num_q_tiles - 1 - bx;  // latest (heaviest) tiles first
  const int kvh = by, seq = bz;
  const int q_begin = p.cu_seq_q[seq], q_end = p.cu_seq_q[seq + 1];
  const int nq = q_end - q_begin, nk = p.cu_seq_k[seq + 1] - p.cu_seq_k[seq];
  const int t0 = tile * p.q_tile;
  if (t0 >= nq) return;
  const int t1 = min(t0 + p.q_tile, nq);

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  QT *out = reinterpret_cast<QT *>(p.out);

  // Column j of the wave: (query token, query head) pair 64 wv + 16 j + n.
  int tok[NT], head[NT], vlo[NT], vhi[NT];
  bool col_ok[NT];
  const long long pos0 = (long long)nk - nq;  // position of query token 0
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int col = 16 * (NT * wv + j) + n;
    tok[j] = t0 + col / p.group;
    head[j] = kvh * p.group + col % p.group;
    col_ok[j] = col < p.q_tile * p.group && tok[j] < t1;
    // The keys this column sees: [vlo, vhi).
    const long long qpos = pos0 + tok[j];
    long long a = 0, b = nk;
    if (p.causal) b = min(b, qpos + 1);
    if (p.window_right >= 0) b = min(b, qpos + 1 + p.window_right);
    if (p.window_left >= 0) a = max(a, qpos - p.window_left);
    vlo[j] = col_ok[j] ? (int)max(a, 0LL) : 0;
    vhi[j] = col_ok[j] ? (int)max(min(b, (long long)nk), 0LL) : 0;
  }

  // Lengths or offsets the host could not check: the tile's rows become NaN.
  const bool bad = nk < 0 || nk > p.max_seq_k || nq > p.max_seq_q || q_begin < 0 ||
                   q_end > p.total_q;
  if (bad) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (col_ok[j] && q_begin >= 0 && q_begin + tok[j] < p.total_q) {
        QT *row = out + ((size_t)(q_begin + tok[j]) * p.num_heads + head[j]) * D;
        for (int d = 4 * g; d < D; d += 16)
          for (int e = 0; e < 4; ++e) row[d + e] = from_f32<QT>(__builtin_nanf(""));
      }
    }
    return;
  }

  // Keys any column of the workgroup sees.
  long long lo = 0, hi = nk;
  if (p.causal) hi = min(hi, pos0 + t1);
  if (p.window_right >= 0) hi = min(hi, pos0 + t1 + p.window_right);
  if (p.window_left >= 0) lo = max(lo, pos0 + t0 - p.window_left);

  // B operands of QK^T: 8 query values per lane, column tile and k-step.
  u32x4 qop[NT][NKS];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const QT *q = reinterpret_cast<const QT *>(p.query) +
                  ((size_t)(q_begin + (col_ok[j] ? tok[j] : t0)) * p.num_heads + head[j]) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qop[j][ks] = col_ok[j] ? load16(q + 32 * ks + 8 * g) : u32x4{0u, 0u, 0u, 0u};
  }

  const char *kcache = reinterpret_cast<const char *>(p.key_cache);
  const char *vcache = reinterpret_cast<const char *>(p.value_cache);
  const const_i32_ptr btab =
      as_const_table(p.block_tables + (size_t)seq * p.max_num_blocks_per_seq);
  // An out-of-range table entry reads block 0 and poisons the workgroup's
  // result.
  const size_t head_off = (size_t)kvh * BS * D * sizeof(QT);
  const size_t blk_stride = (size_t)p.num_kv_heads * BS * D * sizeof(QT);
  bool poisoned = false;

  // The reference starts at the lowest finite float rather than -inf, so
  // that x - m_run is -inf, and its weight 0, for a masked logit whatever
  // the column has seen (with -inf it would be NaN before the first move).
  // Without a cap, m_thr is the raw dot product above which a logit exceeds
  // the reference by more than the lazy margin, (m_run + margin) /
  // scale_log2 (scale_log2 >= 0; infinite for a zero scale), so that a step
  // compares its raw maxima without scaling them.
  const float inv_scale_log2 = 1.0f / p.scale_log2;
  float m_run[NT], l_run[NT], m_thr[NT];
  f32x4 oacc[NT][NDT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    m_thr[j] = -__builtin_inff();
    m_run[j] = -__FLT_MAX__;
    l_run[j] = 0.0f;
#pragma unroll
    for (int t = 0; t < NDT; ++t) oacc[j][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Per lane: base of the QK operand reads and of the
  // transposing V reads.  Row 4 q + e of a 16-key sub-tile h of the QK
  // product is key 16 h + 4 tau(q) + e (tau a permutation of the four
  // 4-key groups), and the PV product pairs contraction index 8 g + 4 r + m
  // of lane group g with key 16 r + 4 tau(g) + m: exactly the keys whose
  // weights the lane holds from the QK product (rows 4 g + m of sub-tile r),
  // so P is used as computed, with no lane exchange.  In a transposing
  // read, lane 4 m + x of group g names key 16 r + 4 tau(g) + m, dims 4 x
  // of a 16-dim tile.  A 64-lane transposing read is served 32 lanes at a
  // time, so lane groups 0 and 1 (and 2 and 3) must fall on disjoint banks:
  // with 128 dims (successive loads a quarter of the banks apart) tau swaps
  // the two bits of the group, which puts them half the banks apart; with 64
  // dims the groups already alternate within a load.  The K reads (16 lanes
  // at a time) stay conflict free under either.
  auto ring_tau = [](int q) { return RG::KPI == 4 ? (((q & 1) << 1) | (q >> 1)) : q; };
  const int krow = 4 * ring_tau(n >> 2) + (n & 3);
  const int koff = (krow / RG::KPI) * RG::IB + 16 * (RG::KPI * g + krow % RG::KPI);
  const int vkey = 4 * ring_tau(g) + (n >> 2);
  // Key of element e of sub-tile h in this lane's QK output: base + 16 h +
  // kgrp + e.
  const int kgrp = 4 * ring_tau(g);
  const int voff = (vkey / RG::KPI) * RG::IB + 16 * (RG::KPI * ((n >> 1) & 1) + vkey % RG::KPI) +
                   8 * (n & 1);
  // The keys every valid column of the wave sees: [full_lo, full_hi)
  // (wave-uniform; a wave without valid columns sees everything).
  int full_lo, full_hi;
  {
    int a = -1, b = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NT; ++j)
      if (col_ok[j]) {
        a = max(a, vlo[j]);
        b = min(b, vhi[j]);
      }
    full_lo = wave_max32(a);
    full_hi = -wave_max32(-b);
  }
  // first: the wave's first step, whose accumulators are still zero (a
  // rescale of them would change nothing).
  auto compute = [&](int base, const char *kst, bool first) {
    // Every valid column of the wave sees the whole step: no masks needed.
    const bool full = base >= full_lo && base + kPrefillStep <= full_hi;
    // S^T of every column tile; each K fragment read from LDS feeds NT MFMAs.
    f32x4 sc[NT][NSUB];
#pragma unroll
    for (int h = 0; h < NSUB; ++h)
#pragma unroll
      for (int j = 0; j < NT; ++j) sc[j][h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int h = 0; h < NSUB; ++h) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(kst + koff + h * (16 / RG::KPI) * RG::IB +
                                                         64 * RG::KPI * ks);
#pragma unroll
        for (int j = 0; j < NT; ++j) sc[j][h] = mfma_qk(a, qop[j][ks], sc[j][h], QT());
      }
    }
    u32x4 pop[NT][NHALF];
    // P of column tile j from its logits (x = log2-domain logit, or the raw
    // dot product when RAW): weights exp2(x - m_run), rounded to the 16-bit
    // P operand; l_run accumulates the rounded weights (the ones the PV
    // product uses), two at a time with a dot product against (1, 1).
    auto make_p = [&](int j, auto raw, const float (&x)[NSUB][4]) {
      u32x2 pk[NSUB];
#pragma unroll
      for (int h = 0; h < NSUB; ++h) {
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (decltype(raw)::value)
            pe[e] = fast_exp2(fmaf(x[h][e], p.scale_log2, -m_run[j]));
          else
            pe[e] = fast_exp2(x[h][e] - m_run[j]);
        }
        pk[h] = u32x2{pack2(pe[0], pe[1], QT()), pack2(pe[2], pe[3], QT())};
        l_run[j] = dot2_sum(pk[h].x, dot2_sum(pk[h].y, l_run[j], QT()), QT());
      }
#pragma unroll
      for (int hf = 0; hf < NHALF; ++hf)
        pop[j][hf] = u32x4{pk[2 * hf].x, pk[2 * hf].y, pk[2 * hf + 1].x, pk[2 * hf + 1].y};
    };
    // Moves column j's reference to bm when bm exceeds it by more than the
    // lazy margin, rescaling its sum and accumulators (the initial reference
    // moves for any finite bm above the lowest float: alpha 0, and l_run and
    // oacc are 0).  Returns the factor.
    auto move_ref = [&](int j, float bm) {
      const bool move = bm > m_run[j] + kLazyRescale;
      const float alpha = move ? fast_exp2(m_run[j] - bm) : 1.0f;
      m_run[j] = move ? bm : m_run[j];
      if constexpr (!CAP) m_thr[j] = move ? (bm + kLazyRescale) * inv_scale_log2 : m_thr[j];
      l_run[j] *= alpha;
      return alpha;
    };
    float alpha[NT];
    bool moved;  // some column's reference moved (wave-uniform)
    if constexpr (!CAP) {
      // No cap (and scale_log2 > 0: a zero scale runs the capped form): the
      // logits are the raw dot products scaled once, inside the weights'
      // fma, and a masked key's raw value becomes -inf, whose weight is 0.
      // Full and masked steps then share one path, and the softmax state
      // one set of registers.  Each lane first checks its own raw maxima
      // against the columns' thresholds; only when some lane's exceed them
      // (the first steps, then rarely) does the wave take the column maxima
      // across lanes and move references.
      if (!full) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int h = 0; h < NSUB; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = base + 16 * h + kgrp + e;
              if (t < vlo[j] || t >= vhi[j]) sc[j][h][e] = -__builtin_inff();
            }
      }
      float lm[NT];
      bool need = false;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        float v = -__builtin_inff();
#pragma unroll
        for (int h = 0; h < NSUB; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) v = fmaxf(v, sc[j][h][e]);
        lm[j] = v;
        need |= v > m_thr[j];
      }
      moved = false;
      if (__any(need)) {
        moved = true;
        // A column with nothing visible yet has max -inf and does not move.
#pragma unroll
        for (int j = 0; j < NT; ++j)
          alpha[j] = move_ref(j, xor_max<32>(xor_max<16>(lm[j])) * p.scale_log2);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        float x[NSUB][4];
#pragma unroll
        for (int h = 0; h < NSUB; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[h][e] = sc[j][h][e];
        make_p(j, std::true_type(), x);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        float x[NSUB][4];
        float bm = -__builtin_inff();
#pragma unroll
        for (int h = 0; h < NSUB; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = base + 16 * h + kgrp + e;
            const float v = scaled_logit<CAP>(p, sc[j][h][e]);
            x[h][e] = (full || (t >= vlo[j] && t < vhi[j])) ? v : -__builtin_inff();
            bm = fmaxf(bm, x[h][e]);
          }
        // bm = -inf (nothing visible yet) never moves the reference.
        alpha[j] = move_ref(j, xor_max<32>(xor_max<16>(bm)));
        make_p(j, std::false_type(), x);
      }
      bool same = true;
#pragma unroll
      for (int j = 0; j < NT; ++j) same &= alpha[j] == 1.0f;
      moved = !__all(same);
    }
    // Rescale the accumulators only when some column's reference moved.
    if (moved && !first) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int t = 0; t < NDT; ++t) oacc[j][t] = oacc[j][t] * alpha[j];
    }
    // O^T += V^T . P^T per 32-key slice; each V fragment read from LDS feeds
    // NT MFMAs.
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int hf = 0; hf < NHALF; ++hf) {
        const char *rd = kst + RG::TILE + voff + hf * (32 / RG::KPI) * RG::IB + 32 * RG::KPI * t;
        const u32x2 lo = lds_read_tr16(rd);
        const u32x2 hi = lds_read_tr16(rd + (16 / RG::KPI) * RG::IB);
        const u32x4 va = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int j = 0; j < NT; ++j) oacc[j][t] = mfma_pv(va, pop[j][hf], oacc[j][t], QT());
      }
    }
  };

  if (threadIdx.x == 0) sm_bad = 0;
  __syncthreads();
  const int base = (int)(lo - lo % BS);  // steps start on a block boundary: earlier blocks are never read
  {
    // Three stages, one barrier per step: at step s the loads of s and
    // s + 1 are in flight; the wave waits for its own loads of s, the
    // barrier publishes everyone's and frees stage s - 1 (every wave has
    // consumed its reads of it), the loads of s + 2 go into that stage, and
    // step s is computed.  The barrier is bracketed by compiler-only
    // fences: a memory fence would make the compiler wait for every load in
    // flight, the prefetched stages included.
    const int n_steps = base < hi ? (int)((hi - base + kPrefillStep - 1) / kPrefillStep) : 0;
    // Lane l of a load fetches chunk l / KPI of key l % KPI of a 1 KB run of
    // KPI keys; a wave's IPW loads cover 8 consecutive keys of one block.
    const int loff = (lane % RG::KPI) * RG::ROWB + 16 * (lane / RG::KPI);
    const int kb0 = wv * RG::IPW * RG::KPI;
    auto issue = [&](int sbase, char *st) {
      int phys = 0;
      if (sbase + kb0 < nk) {
        phys = btab[(sbase + kb0) / BS];
        if (phys < 0 || phys >= p.num_blocks) {
          poisoned = true;
          phys = 0;
        }
      }
      const size_t blk = (size_t)phys * blk_stride + head_off + (size_t)(kb0 % BS) * RG::ROWB;
#pragma unroll
      for (int ii = 0; ii < RG::IPW; ++ii) {
        const int i = wv * RG::IPW + ii;
        const unsigned lds = lds_addr(st) + i * RG::IB;
        lds_dma16(kcache + blk + 1024 * ii + loff, __builtin_amdgcn_readfirstlane(lds));
        lds_dma16(vcache + blk + 1024 * ii + loff,
                  __builtin_amdgcn_readfirstlane(lds + RG::TILE));
      }
    };
    // The stage of step s is s % 3, kept as a byte offset in a scalar.
    int cur_off = 0;
    if (n_steps > 0) issue(base, ring);
    // A use of the query registers here makes the compiler wait for the
    // query loads (and with them stage 0, needed first anyway) before the
    // loop, inside which it then has no load of its own to wait for.
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(qop[j][ks]));
    if (n_steps > 1) issue(base + kPrefillStep, ring + RG::STAGE);
    for (int s = 0; s < n_steps; ++s) {
      if (s + 1 < n_steps)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * RG::IPW));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int ahead_off = cur_off == 0 ? 2 * RG::STAGE : cur_off - RG::STAGE;
      if (s + 2 < n_steps) issue(base + kPrefillStep * (s + 2), ring + ahead_off);
      const int sbase = base + kPrefillStep * s;
      char *const cur = ring + cur_off;
      if (sbase + kPrefillStep > nk) {
        // The step runs past the last key: those rows hold whatever the
        // cache holds there, and a zero weight times a NaN is NaN, so their
        // V rows are zeroed before anyone reads the stage.
        char *vt = cur + RG::TILE;
        for (int c = threadIdx.x; c < kPrefillStep * (D / 8); c += kThreads) {
          const int key = c / (D / 8), ch = c % (D / 8);
          if (sbase + key >= nk)
            *reinterpret_cast<u32x4 *>(vt + (key / RG::KPI) * RG::IB +
                                       16 * (RG::KPI * ch + key % RG::KPI)) =
                u32x4{0u, 0u, 0u, 0u};
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the stores are done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      compute(sbase, cur, s == 0);
      cur_off = cur_off == 2 * RG::STAGE ? 0 : cur_off + RG::STAGE;
    }
  }
  if (poisoned) sm_bad = 1;
  __syncthreads();

  const bool nan_out = sm_bad != 0;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const float l_tot = xor_sum<32>(xor_sum<16>(l_run[j]));
    if (!col_ok[j]) continue;
    QT *row = out + ((size_t)(q_begin + tok[j]) * p.num_heads + head[j]) * D;
    // One reciprocal per column (the output is rounded to 16 bits).
    const float inv = nan_out ? __builtin_nanf("") : (l_tot > 0.0f ? 1.0f / l_tot : 0.0f);
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = oacc[j][t][e] * inv;
      *reinterpret_cast<u32x2 *>(row + 16 * t + 4 * g) =
          u32x2{pack2(o[0], o[1], QT()), pack2(o[2], o[3], QT())};
    }
  }
}

template <typename QT, int D, int BS>
static hipError_t launch_prefill_bs(const PrefillParams &p, bool cap, const Launch &l) {
  if (p.tiles_per_wave == 2)
    return cap ? launch_kernel(pa_prefill_kernel<QT, D, BS, 2, true>, l, p)
               : launch_kernel(pa_prefill_kernel<QT, D, BS, 2, false>, l, p);
  return cap ? launch_kernel(pa_prefill_kernel<QT, D, BS, 1, true>, l, p)
             : launch_kernel(pa_prefill_kernel<QT, D, BS, 1, false>, l, p);
}

template <typename QT>
static hipError_t launch_prefill_t(const PrefillParams &p, int head_size, int block_size,
                                   bool cap, const Launch &l) {
  if (head_size == 64 && block_size == 16) return launch_prefill_bs<QT, 64, 16>(p, cap, l);
  if (head_size == 64 && block_size == 32) return launch_prefill_bs<QT, 64, 32>(p, cap, l);
  if (head_size == 128 && block_size == 16) return launch_prefill_bs<QT, 128, 16>(p, cap, l);
  if (head_size == 128 && block_size == 32) return launch_prefill_bs<QT, 128, 32>(p, cap, l);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_size, int block_size,
                          bool cap, const Launch &l) {
  if (dtype == kDtF16) return launch_prefill_t<_Float16>(p, head_size, block_size, cap, l);
  if (dtype == kDtBF16) return launch_prefill_t<__bf16>(p, head_size, block_size, cap, l);
  return hipErrorInvalidValue;
}

}  // namespace pa
