// Work decoding and the cross-wave merge / store epilogue shared by the two
// partition-phase kernels (VALU and MFMA).
//
// Grid: x = KV head * head_groups + head group, y = sequence, z = partition
// (v2) or 0 (v1).  Each workgroup owns one (sequence, KV head, query-head
// group) and either one 512-token partition (v2) or the whole sequence (v1).
// The partition is the slowest grid dimension.  A launch that mixes v1 and v2
// dispatches partition 0 first, so its long whole-sequence workgroups start
// early instead of queueing behind the empty partition slots of their
// sequence.  A launch whose sequences all take v2 dispatches the last
// partition first: the grid slices of high partitions, mostly empty slots of
// the shorter sequences, pass while the device fills, and the launch ends on
// partition 0, full for every sequence, instead of on a few long-sequence
// workgroups that cannot keep HBM busy.
#pragma once

#include "pa_device.h"
#include "pa_merge.h"
#include "pa_worklist.h"

namespace pa {

struct Work {
  int seq, kvh, head0, nh;  // sequence, KV head, first query head, query heads in the group
  int xslot;                // grid-x slot (KV head x head group)
  int L, n_part, part;      // sequence length, its partitions, this workgroup's partition
  int blk_begin, blk_end;   // logical blocks [blk_begin, blk_end) of this workgroup
  int t_ref;                // last token of this workgroup's range (ALiBi reference)
  int t_lo, span;           // keys weighed: [t_lo, t_lo + span) = window start .. t_ref
  bool v2;                  // partials are stored (v2) or out is written directly (v1)
  bool single;              // v2 with one partition in the window: out is written too
};

// threadIdx.x for the epilogues, through an empty asm statement: in the
// persistent list form the epilogue runs once per item, and without this the
// compiler hoists its thread-dependent addresses out of the item loop and
// spills them.  (No instruction is emitted; the value is the thread index.)
__device__ __forceinline__ int epi_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

template <typename QT, int D>
__device__ __forceinline__ void store_out_row(const Params &p, int seq, int head, int d, float v) {
  QT *out = reinterpret_cast<QT *>(p.out);
  out[((size_t)seq * p.num_heads + head) * D + d] = from_f32<QT>(v);
}

// Partition slots a sequence does not use hold max_logit = -inf and
// exp_sum = 0 (page "BI-V100 PagedAttention V2 implementation", the step
// that zeroes out unused partitions).  tmp_out of those slots is not written.
__device__ __forceinline__ void write_stat_padding(const Params &p, const Work &w, int first) {
  const int count = p.max_num_partitions - first;
  for (int idx = threadIdx.x; idx < w.nh * count; idx += kThreads) {
    const int h = idx / count, slot = first + (idx - h * count);
    const size_t row = ((size_t)w.seq * p.num_heads + w.head0 + h) * p.max_num_partitions + slot;
    p.max_logits[row] = -__builtin_inff();
    p.exp_sums[row] = 0.0f;
  }
}

// The statistics of one partition slot with no key in the window: the
// padding values, no tmp_out row.
__device__ __forceinline__ void write_stat_empty(const Params &p, const Work &w, int slot) {
  if (threadIdx.x < w.nh) {
    const size_t row =
        ((size_t)w.seq * p.num_heads + w.head0 + threadIdx.x) * p.max_num_partitions + slot;
    p.max_logits[row] = -__builtin_inff();
    p.exp_sums[row] = 0.0f;
  }
}

// Decodes one work item (sequence, grid-x slot = KV head x head group,
// partition) into a Work.  Returns false when there is nothing (more) to
// compute; sequences of length 0 (out = 0) and with an invalid length
// (out = NaN) are finished here by their partition-0 item.  Under a sliding
// window the range starts at the block holding the first key of the window;
// v2 partitions before it only store padding statistics.
template <typename QT, int D>
__device__ __forceinline__ bool decode_work(const Params &p, int seq, int xslot, int part,
                                           int block_size, int group_slots, Work &w) {
  w.seq = seq;
  w.xslot = xslot;
  w.kvh = xslot / p.head_groups;
  const int hg = xslot - w.kvh * p.head_groups;
  w.head0 = w.kvh * p.group + hg * group_slots;
  w.nh = min(group_slots, p.group - hg * group_slots);
  w.L = p.seq_lens[w.seq];
  const bool bad = (w.L < 0) || (w.L > p.max_seq_len);
  w.t_lo = bad ? 0 : window_first_token(p.window_left, w.L);
  const bool split = p.mode == kModeSplit;
  w.v2 = !split && seq_uses_v2(p, bad ? 0 : w.L - w.t_lo);
  w.single = false;
  w.n_part = bad ? 0 : (w.L + kPartitionSize - 1) / kPartitionSize;
  w.part = part;
  if (bad || w.L == 0) {
    if (w.part != 0) return false;
    const float fill = bad ? __builtin_nanf("") : 0.0f;
    for (int idx = threadIdx.x; idx < w.nh * D; idx += kThreads)
      store_out_row<QT, D>(p, w.seq, w.head0 + idx / D, idx % D, fill);
    if (w.v2) {
      write_stat_padding(p, w, bad ? 1 : 0);
      if (bad && threadIdx.x < w.nh) {
        const size_t row =
            ((size_t)w.seq * p.num_heads + w.head0 + threadIdx.x) * p.max_num_partitions;
        p.max_logits[row] = __builtin_nanf("");
        p.exp_sums[row] = __builtin_nanf("");
      }
    }
    return false;
  }
  const int n_logical = (w.L + block_size - 1) / block_size;
  if (split) {
    // Pieces start on 32-key boundaries from the window's first aligned key;
    // every piece but a sequence's only one spans at least 512 keys, so
    // grid slices past len / 512 are empty without further work.
    const int base = w.t_lo / 32 * 32;
    const int len = w.L - base;
    if (w.part * 512 >= len) return false;
    // k = ceil(len / split_target) pieces (at most the grid's depth) of
    // equal length rounded up to 32 keys.
    const int piece = split_piece_len(p.split_target, len, (int)gridDim.z);
    const int k = (len + piece - 1) / piece;
    if (w.part >= k) return false;
    w.n_part = k;
    w.v2 = k > 1;  // partials, merged by the last piece to finish
    const int t0 = base + w.part * piece, t1 = min(t0 + piece, w.L);
    w.blk_begin = max(t0, w.t_lo) / block_size;
    w.blk_end = (t1 + block_size - 1) / block_size;
    w.t_ref = t1 - 1;
  } else if (w.v2) {
    if (w.part >= w.n_part) return false;
    if (w.part == 0) write_stat_padding(p, w, w.n_part);
    const int part_lo = w.t_lo / kPartitionSize;  // first partition with a key in the window
    if (w.part < part_lo) {
      write_stat_empty(p, w, w.part);
      return false;
    }
    w.single = w.n_part - part_lo == 1;
    const int bpp = kPartitionSize / block_size;
    w.blk_begin = max(w.part * bpp, w.t_lo / block_size);
    w.blk_end = min(w.part * bpp + bpp, n_logical);
    w.t_ref = min((w.part + 1) * kPartitionSize, w.L) - 1;
  } else {
    if (w.part != 0) return false;
    w.blk_begin = w.t_lo / block_size;
    w.blk_end = n_logical;
    w.t_ref = w.L - 1;
  }
  // The upper bound matters where a 32-token MFMA step that starts inside
  // the window's first block runs past the end of a v2 partition.
  w.span = w.t_ref + 1 - w.t_lo;
  return true;
}

// One item per workgroup: (x, y, z) = (slot, sequence, partition), the
// partition counted from the last one when parts_reversed is set.
template <typename QT, int D>
__device__ __forceinline__ bool begin_work(const Params &p, int block_size, int group_slots,
                                          Work &w) {
  const int part = p.parts_reversed ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z;
  return decode_work<QT, D>(p, blockIdx.y, blockIdx.x, part, block_size, group_slots, w);
}

// ---------------------------------------------------------------------------
// Split mode: the pieces of one (sequence, grid-x slot) exchange their
// partials through memory and an arrival counter.  The partials are stored
// and loaded with agent-scope relaxed atomics, which gfx950 performs at
// device scope (`global_store` / `global_load` with sc1: written through
// and read past the per-XCD L2 caches).  Every wave of a piece waits for
// its partial stores to be performed (s_waitcnt vmcnt(0)) and meets the
// others at a barrier; then one lane adds 1 to the counter with the
// device-scope atomic add the compiler emits for an agent-scope fetch-add.
// The piece that reads k - 1 from it issues the merge's loads only after
// that value has returned (they depend on it), and they read the device
// coherence point, so they see every other piece's partials: each of those
// was performed before that piece's increment was issued.  The HIP memory
// model would express the same ordering as a release increment and an
// acquire in the merging piece (PA_ARRIVE_RELEASE_ACQUIRE = 1), which
// gfx950 lowers to an L2 writeback before every increment and an L2
// invalidate in every merging piece: nothing for accesses that bypass the
// L2 anyway, but they measured 2-3% on cut batches (ragged ALiBi split
// 2134 vs 2074 us, work list 2079 vs 2037 us) and far more where many
// items are cut, so the default relies on the device-scope accesses above.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void coherent_store(void *ptr, unsigned v) {
  __hip_atomic_store(reinterpret_cast<unsigned *>(ptr), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned coherent_load(const void *ptr) {
  return __hip_atomic_load(reinterpret_cast<const unsigned *>(ptr), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// One element of a partial row, rounded to QT (fp32 or a 16-bit type),
// stored / loaded past the L2.
template <typename QT>
__device__ __forceinline__ void coherent_store_elem(QT *ptr, float v) {
  if constexpr (sizeof(QT) == 4) {
    coherent_store(ptr, f_bits(v));
  } else {
    __hip_atomic_store(reinterpret_cast<unsigned short *>(ptr),
                       __builtin_bit_cast(unsigned short, from_f32<QT>(v)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}
template <typename QT>
__device__ __forceinline__ float coherent_load_elem(const QT *ptr) {
  if constexpr (sizeof(QT) == 4) {
    return bits_f(coherent_load(ptr));
  } else {
    return to_f32(__builtin_bit_cast(
        QT, __hip_atomic_load(reinterpret_cast<const unsigned short *>(ptr), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT)));
  }
}

// Four consecutive values of a partial row (fp32, or the 16-bit type TT),
// read past the L2 with 8-byte agent-scope loads (ptr 8-byte aligned): the
// raw bits, then the values.
struct Raw4 {
  unsigned long long a, b;
};
__device__ __forceinline__ unsigned long long coherent_load8(const void *ptr) {
  return __hip_atomic_load(reinterpret_cast<const unsigned long long *>(ptr), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
template <typename TT>
__device__ __forceinline__ Raw4 coherent_load4(const TT *ptr) {
  if constexpr (sizeof(TT) == 4) return Raw4{coherent_load8(ptr), coherent_load8(ptr + 2)};
  else return Raw4{coherent_load8(ptr), 0ull};
}
template <typename TT>
__device__ __forceinline__ void unpack4(const Raw4 &r, float (&v)[4]) {
  if constexpr (sizeof(TT) == 4) {
    v[0] = bits_f((unsigned)r.a);
    v[1] = bits_f((unsigned)(r.a >> 32));
    v[2] = bits_f((unsigned)r.b);
    v[3] = bits_f((unsigned)(r.b >> 32));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = to_f32(__builtin_bit_cast(TT, (unsigned short)(r.a >> (16 * e))));
  }
}

// The counter operations of the arrival (the ordering is described with
// coherent_store above).  PA_ARRIVE_RELEASE_ACQUIRE = 1: agent-scope release
// increment and acquire load; 0 (default): relaxed increment, no acquire.
#ifndef PA_ARRIVE_RELEASE_ACQUIRE
#define PA_ARRIVE_RELEASE_ACQUIRE 0
#endif
__device__ __forceinline__ int arrive_add(int *c) {
  return __hip_atomic_fetch_add(c, 1, PA_ARRIVE_RELEASE_ACQUIRE ? __ATOMIC_RELEASE : __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void arrive_acquire(int *c) {
  if constexpr (PA_ARRIVE_RELEASE_ACQUIRE)
    (void)__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void arrive_reset(int *c, int v) {
  __hip_atomic_store(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Four values in the raw form coherent_load4 returns for a TT row: the
// values rounded to TT, as a stored partial would hold them.
template <typename TT>
__device__ __forceinline__ Raw4 pack4(const float (&v)[4]) {
  if constexpr (sizeof(TT) == 4) {
    return Raw4{(unsigned long long)f_bits(v[0]) | ((unsigned long long)f_bits(v[1]) << 32),
                (unsigned long long)f_bits(v[2]) | ((unsigned long long)f_bits(v[3]) << 32)};
  } else {
    unsigned long long a = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a |= (unsigned long long)__builtin_bit_cast(unsigned short, from_f32<TT>(v[e])) << (16 * e);
    return Raw4{a, 0ull};
  }
}

__device__ __forceinline__ int *item_counter(const Params &p, int seq, int xslot) {
  return p.counters + (size_t)seq * p.num_heads + xslot;
}

// The Phase 2 merge (V2 page, "Phase 2: Reduce across partitions") of the k
// pieces of item (seq, heads head0 .. head0 + nh - 1) into out, by the whole
// workgroup.  Piece c's partials are read from its slot c, past the L2,
// except piece `own` (>= 0), whose normalised rows are own_o[h][d] and
// statistics own_m[h] (max logit, absolute) / own_s[h] (exp-sum) in LDS;
// they are rounded to the partial type as a stored partial would be, so the
// result does not depend on which piece merges.  Ends with the out stores
// issued.
// The merge's statistics in LDS: one copy per kernel, whatever the
// instantiations of merge_pieces it holds.
struct MergeLds {
  float pm[16][kSplitMaxPieces], ps[16][kSplitMaxPieces], sum[16];
};
__device__ __forceinline__ MergeLds &merge_lds() {
  __shared__ MergeLds m;
  return m;
}

template <typename QT, typename TT, int D, int OSTRIDE>
__device__ __forceinline__ void merge_pieces(const Params &p, int seq, int head0, int nh, int k,
                                             int own, const float (*own_o)[OSTRIDE],
                                             const float *own_m, const float *own_s) {
  MergeLds &ml = merge_lds();
  auto &sm_pm = ml.pm;
  auto &sm_ps = ml.ps;
  auto &sm_sum = ml.sum;
  const int tid = epi_tid();
  // At most kSplitMaxPieces pieces by construction (every piece mode); the
  // bound keeps the LDS statistics in range whatever the caller's sizes.
  k = min(k, kSplitMaxPieces);
  const size_t row0 = ((size_t)seq * p.num_heads + head0) * p.max_num_partitions;
  for (int idx = tid; idx < nh * k; idx += kThreads) {
    const int h = idx / k, c = idx - h * k;
    const size_t r = row0 + (size_t)h * p.max_num_partitions + c;
    float m, sv;
    if (c == own) {
      m = own_m[h];
      sv = own_s[h];
    } else {
      const unsigned m_bits = coherent_load(p.max_logits + r);
      const unsigned s_bits = coherent_load(p.exp_sums + r);
      m = bits_f(m_bits);
      sv = bits_f(s_bits);
    }
    sm_pm[h][c] = m;
    sm_ps[h][c] = sv;
  }
  __syncthreads();
  // Per head: the rescaled exp-sums r_c, in place of S_c, and their sum.
  if (tid < nh)
    sm_sum[tid] = lse_rescale(
        [&](int c) { return sm_pm[tid][c]; }, [&](int c) { return sm_ps[tid][c]; }, k,
        [](float x) { return fast_exp2(x); }, [&](int c, float r) { sm_ps[tid][c] = r; });
  __syncthreads();
  // Per thread: four consecutive dims of one head, all pieces' slices requested at once.
  constexpr int G = D / 4;
  const TT *to = reinterpret_cast<const TT *>(p.tmp_out);
  for (int idx = tid; idx < nh * G; idx += kThreads) {
    const int h = idx / G, d0 = 4 * (idx - h * G);
    const TT *col = to + (row0 + (size_t)h * p.max_num_partitions) * D + d0;
    float o[4];
    lse_combine<4>(
        [&](int c) { return sm_ps[h][c]; }, sm_sum[h], k,
        [&](int c) {
          if (c == own) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = own_o[h][d0 + e];
            return pack4<TT>(v);
          }
          return coherent_load4<TT>(col + (size_t)c * D);
        },
        [](const Raw4 &r, float(&v)[4]) { unpack4<TT>(r, v); }, o);
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out_row<QT, D>(p, seq, head0 + h, d0 + e, o[e]);
  }
}

// After a piece's partials are stored (slot = piece): the piece that
// arrives last at the (sequence, grid-x slot) counter merges the k pieces
// with the log-sum-exp rescale of the V2 page's Phase 2, writes out, and
// resets the counter to zero for the next call.
template <typename QT, typename TT, int D>
__device__ __forceinline__ void split_merge(const Params &p, const Work &w) {
  __shared__ int sm_last;
  const int tid = epi_tid();
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are done
  __syncthreads();
  if (tid == 0) {
    sm_last = arrive_last(
        item_counter(p, w.seq, w.xslot), w.n_part,
        [](int *c) { return arrive_add(c); }, [](int *c) { arrive_acquire(c); },
        [](int *c, int v) { arrive_reset(c, v); });
  }
  __syncthreads();
  if (!sm_last) return;
  merge_pieces<QT, TT, D, 4>(p, w.seq, w.head0, w.nh, w.n_part, -1, nullptr, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// List mode (paged_attention_worklist): a persistent launch in which every
// wave is a worker.  The batch's items -- (sequence, grid-x slot) -- lie end
// to end on a line by their memory-load cost (pa_worklist.h); worker w takes
// the w-th equal share of the line, with its ends snapped so that an item is
// cut only on 32-key steps and at least 512 keys from its ends.  Every
// worker builds its own part of the list: it scans seq_lens with wave-wide
// prefix sums, finds the items holding its two boundaries, and then walks
// the items in between, each one whole, with its own online softmax.  Its
// epilogue works from registers: a whole item writes out; a cut item's piece
// stores its partials in its slot and arrives at the item's counter, and the
// last piece to arrive merges them.  No step of it waits for the other waves
// of the workgroup, so one wave's epilogue overlaps the others' streaming.
// ---------------------------------------------------------------------------
struct ListCursor {
  ListShares sh;     // line length T, workers with work W, the equal shares
  int w;             // this worker
  long long end;     // snapped end of this worker's range on the line
  long long pos;     // line position of the current item
  int seq, x;        // current item
  int L, keys, base; // its length, keys on the line, first key (32-aligned window start)
  int L_next;        // length of sequence seq + 1 (read one sequence ahead; 0 past the batch)
  long long cost;
  long long start;   // offset at which this worker's piece of the current item starts
};

// Lane l's 64-bit value (l wave-uniform), as a scalar.
__device__ __forceinline__ long long readlane64(long long v, int l) {
  const unsigned lo = __builtin_amdgcn_readlane((unsigned)(unsigned long long)v, l);
  const unsigned hi = __builtin_amdgcn_readlane((unsigned)((unsigned long long)v >> 32), l);
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Wave-uniform 64-bit value (every lane holds the same).
__device__ __forceinline__ long long wave_uniform64(long long v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long long)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ int uniform32(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ long long wave_sum64(long long v) {
#pragma unroll
  for (int m = 1; m < 64; m *= 2) v += __shfl_xor(v, m);
  return wave_uniform64(v);
}

__device__ __forceinline__ int wave_max32(int v) {
#pragma unroll
  for (int m = 1; m < 64; m *= 2) v = max(v, __shfl_xor(v, m));
  return __builtin_amdgcn_readfirstlane(v);
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ long long wave_inclusive_scan64(long long v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const long long t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

// The cursor and a work item hold wave-uniform values; some come out of
// VALU arithmetic (the double quotients of the list geometry), so they are
// moved back to scalar registers: kept in vector registers they would make
// the block-table reads vector loads and crowd the tile registers.
__device__ __forceinline__ void scalarize(ListCursor &c) {
  c.sh.total = wave_uniform64(c.sh.total);
  c.sh.q = wave_uniform64(c.sh.q);
  c.sh.r = wave_uniform64(c.sh.r);
  c.sh.workers = uniform32(c.sh.workers);
  c.end = wave_uniform64(c.end);
  c.pos = wave_uniform64(c.pos);
  c.cost = wave_uniform64(c.cost);
  c.start = wave_uniform64(c.start);
  c.w = uniform32(c.w);
  c.seq = uniform32(c.seq);
  c.x = uniform32(c.x);
  c.L = uniform32(c.L);
  c.L_next = uniform32(c.L_next);
  c.keys = uniform32(c.keys);
  c.base = uniform32(c.base);
}

__device__ __forceinline__ void scalarize(Work &w) {
  w.seq = uniform32(w.seq);
  w.kvh = uniform32(w.kvh);
  w.head0 = uniform32(w.head0);
  w.nh = uniform32(w.nh);
  w.xslot = uniform32(w.xslot);
  w.L = uniform32(w.L);
  w.n_part = uniform32(w.n_part);
  w.part = uniform32(w.part);
  w.blk_begin = uniform32(w.blk_begin);
  w.blk_end = uniform32(w.blk_end);
  w.t_ref = uniform32(w.t_ref);
  w.t_lo = uniform32(w.t_lo);
  w.span = uniform32(w.span);
}

// The list cost of sequence s (lane-parallel), with its keys and base.
__device__ __forceinline__ long long list_seq_cost(const Params &p, int s, int &L, int &keys,
                                                   int &base) {
  L = p.seq_lens[s];
  keys = list_keys(L, p.max_seq_len, p.window_left, &base);
  return list_cost(keys, p.item_cost);
}

// Finds the item holding line position target (0 <= target < T): its
// sequence, slot, line position and the target's offset in it.
__device__ __forceinline__ void list_locate(const Params &p, int gx, long long target,
                                            ListCursor &c, long long &offset) {
  const int lane = threadIdx.x & 63;
  long long run = 0;  // line position of the chunk's first sequence
  for (int s0 = 0; s0 < p.num_seqs; s0 += 64) {
    const int s = s0 + lane;
    int L = 0, keys = 0, base = 0;
    const long long cost = s < p.num_seqs ? list_seq_cost(p, s, L, keys, base) : 0;
    const long long span = cost * gx;
    const long long incl = wave_inclusive_scan64(span, lane);
    const long long chunk = wave_uniform64(__shfl(incl, 63));
    if (target < run + chunk || s0 + 64 >= p.num_seqs) {
      const unsigned long long hit = __ballot(s < p.num_seqs && target < run + incl);
      const int l = hit ? __builtin_ctzll(hit) : min(63, p.num_seqs - 1 - s0);
      const long long item0 = wave_uniform64(__shfl(run + incl - span, l));  // line position of (seq, 0)
      c.seq = s0 + l;
      c.L = __builtin_amdgcn_readfirstlane(__shfl(L, l));
      c.L_next = c.seq + 1 < p.num_seqs ? p.seq_lens[c.seq + 1] : 0;
      c.keys = __builtin_amdgcn_readfirstlane(__shfl(keys, l));
      c.base = __builtin_amdgcn_readfirstlane(__shfl(base, l));
      c.cost = wave_uniform64(__shfl(cost, l));
      const long long rel = target - item0;
      c.x = uniform32((int)list_div(rel, c.cost));
      c.x = c.x < gx ? c.x : gx - 1;
      c.pos = item0 + (long long)c.x * c.cost;
      offset = wave_uniform64(target - c.pos);
      return;
    }
    run += chunk;
  }
}

// Moves the cursor to the next item on the line.
__device__ __forceinline__ void list_advance(const Params &p, int gx, ListCursor &c) {
  c.pos += c.cost;
  c.start = 0;
  if (++c.x < gx) return;
  c.x = 0;
  if (++c.seq >= p.num_seqs) return;
  c.L = c.L_next;
  c.keys = list_keys(c.L, p.max_seq_len, p.window_left, &c.base);
  c.cost = list_cost(c.keys, p.item_cost);
  c.L_next = c.seq + 1 < p.num_seqs ? p.seq_lens[c.seq + 1] : 0;
}

// Batches of at most 64 * kListRegChunks sequences: seq_lens is read once,
// lane l holding sequences 64 i + l, and the worker's range is found from
// those registers (no further reads); larger batches scan seq_lens in
// global memory chunk by chunk.
constexpr int kListRegChunks = 4;

__device__ __forceinline__ bool list_begin_regs(const Params &p, ListCursor &c, int worker,
                                                int grid_workers) {
  constexpr int NC = kListRegChunks;
  const int gx = p.num_kv_heads * p.head_groups;
  const int lane = threadIdx.x & 63;
  const int n = p.num_seqs;
  int L[NC], keys[NC], base[NC];
  long long cost[NC], incl[NC];  // incl: line position just past sequence 64 i + lane's items
#pragma unroll
  for (int i = 0; i < NC; ++i) L[i] = 64 * i + lane < n ? p.seq_lens[64 * i + lane] : 0;
  long long run = 0;
  int kmax = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const bool in = 64 * i + lane < n;
    keys[i] = list_keys(L[i], p.max_seq_len, p.window_left, &base[i]);
    cost[i] = in ? list_cost(keys[i], p.item_cost) : 0;
    kmax = in ? max(kmax, keys[i]) : kmax;
    incl[i] = run;
    if (64 * i < n) {  // chunks past the batch stay at its total
      incl[i] = run + wave_inclusive_scan64(cost[i] * gx, lane);
      run = readlane64(incl[i], 63);
    }
  }
  c.sh = list_shares(run, uniform32(list_workers(run, grid_workers, wave_max32(kmax))));
  c.sh.q = wave_uniform64(c.sh.q);
  c.sh.r = wave_uniform64(c.sh.r);
  c.w = worker;
  if (c.w >= c.sh.workers) return false;
  // The item holding line position target: the first sequence whose items
  // end after it.
  auto locate = [&](long long target, long long &offset) {
    int ci = NC - 1, l = 63;
    bool found = false;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const unsigned long long hit = __ballot(64 * i + lane < n && target < incl[i]);
      if (!found && hit) {
        found = true;
        ci = i;
        l = __builtin_ctzll(hit);
      }
    }
    // Lane l of chunk ci (both wave-uniform): scalar reads of its registers.
    long long end_s = 0, cost_s = 1;
    int L_s = 0, keys_s = 0, base_s = 0, L_n = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (i == ci) {
        end_s = readlane64(incl[i], l);
        cost_s = readlane64(cost[i], l);
        L_s = __builtin_amdgcn_readlane(L[i], l);
        keys_s = __builtin_amdgcn_readlane(keys[i], l);
        base_s = __builtin_amdgcn_readlane(base[i], l);
        // The next sequence's length: lane l + 1 of this chunk, or lane 0 of the next.
        L_n = l < 63 ? __builtin_amdgcn_readlane(L[i], l + 1)
                     : (i + 1 < NC ? __builtin_amdgcn_readlane(L[i + 1 < NC ? i + 1 : i], 0) : 0);
      }
    }
    c.seq = uniform32(64 * ci + l);
    c.L = uniform32(L_s);
    c.L_next = c.seq + 1 < n ? uniform32(L_n) : 0;
    c.keys = uniform32(keys_s);
    c.base = uniform32(base_s);
    c.cost = wave_uniform64(cost_s);
    const long long item0 = wave_uniform64(end_s) - c.cost * gx;
    c.x = uniform32((int)list_div(target - item0, c.cost));
    c.x = c.x < gx ? c.x : gx - 1;
    c.pos = item0 + (long long)c.x * c.cost;
    offset = wave_uniform64(target - c.pos);
  };
  if (c.w + 1 >= c.sh.workers) {
    c.end = c.sh.total;
  } else {
    long long off = 0;
    locate(wave_uniform64(list_boundary(c.sh, c.w + 1)), off);
    c.end = wave_uniform64(c.pos + list_snap(off, c.keys, c.cost));
  }
  long long off = 0;
  locate(wave_uniform64(list_boundary(c.sh, c.w)), off);
  c.start = list_snap(off, c.keys, c.cost);
  if (c.start >= c.cost) list_advance(p, gx, c);
  scalarize(c);
  return true;
}

// Sets up worker `worker` of `grid_workers`; false when it has no range (a
// batch too small for every worker).  Wave-uniform.
__device__ __forceinline__ bool list_begin(const Params &p, ListCursor &c, int worker,
                                           int grid_workers) {
  if (p.num_seqs <= 64 * kListRegChunks) return list_begin_regs(p, c, worker, grid_workers);
  const int gx = p.num_kv_heads * p.head_groups;
  const int lane = threadIdx.x & 63;
  long long sum = 0;
  int kmax = 0;
  for (int s0 = 0; s0 < p.num_seqs; s0 += 64) {
    const int s = s0 + lane;
    int L = 0, keys = 0, base = 0;
    if (s < p.num_seqs) {
      sum += list_seq_cost(p, s, L, keys, base);
      kmax = max(kmax, keys);
    }
  }
  const long long total = wave_sum64(sum) * gx;
  c.sh = list_shares(total, uniform32(list_workers(total, grid_workers, wave_max32(kmax))));
  c.sh.q = wave_uniform64(c.sh.q);
  c.sh.r = wave_uniform64(c.sh.r);
  c.w = worker;
  if (c.w >= c.sh.workers) return false;
  // This worker's end: the next worker's start, snapped.
  if (c.w + 1 >= c.sh.workers) {
    c.end = c.sh.total;
  } else {
    long long off = 0;
    list_locate(p, gx, wave_uniform64(list_boundary(c.sh, c.w + 1)), c, off);
    c.end = wave_uniform64(c.pos + list_snap(off, c.keys, c.cost));
  }
  long long off = 0;
  list_locate(p, gx, wave_uniform64(list_boundary(c.sh, c.w)), c, off);
  c.start = list_snap(off, c.keys, c.cost);
  if (c.start >= c.cost) list_advance(p, gx, c);
  scalarize(c);
  return true;
}

// The next piece of this worker's range as a Work, or false at the end.
// Empty and invalid sequences are finished here (out = 0 / NaN, written by
// the worker's lanes) and skipped.
// SLOTS: the slot form of the list (auto without counters): piece j of an
// item goes to partition slot j, and every item of two or more partitions
// stores partials for the reduce kernel, cut or whole.
template <typename QT, int D, bool SLOTS = false>
__device__ __forceinline__ bool list_next(const Params &p, int block_size, int group_slots,
                                          ListCursor &c, Work &w) {
  const int lane = epi_tid() & 63;
  const int gx = p.num_kv_heads * p.head_groups;
  while (c.pos < c.end && c.seq < p.num_seqs) {
    w.seq = c.seq;
    w.xslot = c.x;
    w.kvh = c.x / p.head_groups;
    const int hg = c.x - w.kvh * p.head_groups;
    w.head0 = w.kvh * p.group + hg * group_slots;
    w.nh = min(group_slots, p.group - hg * group_slots);
    w.L = c.L;
    const long long stop = min(c.cost, c.end - c.pos);  // end of the piece (offset)
    const long long start = c.start;
    const long long item_pos = c.pos, cost = c.cost;
    const int keys = c.keys, base = c.base;
    list_advance(p, gx, c);
    if (keys == 0) {
      // Empty (out = 0) or invalid length (out = NaN); the item is never cut.
      const bool bad = w.L != 0;
      for (int idx = lane; idx < w.nh * D; idx += 64)
        store_out_row<QT, D>(p, w.seq, w.head0 + idx / D, idx % D,
                             bad ? __builtin_nanf("") : 0.0f);
      continue;
    }
    if (stop <= start) continue;
    // A piece that spans its whole item is the item (no boundary falls
    // inside it); only the pieces at the ends of a range need the search.
    if (start == 0 && stop >= cost) {
      w.n_part = 1;
      w.part = 0;
    } else {
      list_piece(c.sh, item_pos, keys, c.w, start, &w.n_part, &w.part);
    }
    w.t_lo = window_first_token(p.window_left, w.L);
    if constexpr (SLOTS) w.v2 = keys > kPartitionSize;
    else w.v2 = w.n_part > 1;
    w.single = false;
    const int t0 = base + (int)start;
    const int t1 = min(base + (int)min(stop, (long long)keys), w.L);
    w.blk_begin = max(t0, w.t_lo) / block_size;
    w.blk_end = (t1 + block_size - 1) / block_size;
    w.t_ref = t1 - 1;
    w.span = w.t_ref + 1 - w.t_lo;
    scalarize(c);
    scalarize(w);
    return true;
  }
  return false;
}

// ---------------------------------------------------------------------------
// List mode: the epilogue of one wave's piece, from registers.
// ---------------------------------------------------------------------------

// The slot form: piece 0 of an item of n_part pieces marks the item's
// partition slots n_part .. ceil(L / 512) - 1 empty (max logit -inf, exp
// sum 0: the reduce kernel weighs them 0 and reads no row of them).  Every
// piece of a cut item spans at least kListMinPiece keys, so an item has no
// more pieces than partitions.  Lanes of one wave.
static_assert(kListMinPiece >= kPartitionSize, "pieces must fit the partition slots");
__device__ __forceinline__ void piece_slot_padding(const Params &p, const Work &w, int lane) {
  if (w.part != 0) return;
  const int extra = (w.L + kPartitionSize - 1) / kPartitionSize - w.n_part;
  for (int idx = lane; idx < w.nh * extra; idx += 64) {
    const int h = idx / extra, slot = w.n_part + idx % extra;
    const size_t row = ((size_t)w.seq * p.num_heads + w.head0 + h) * p.max_num_partitions + slot;
    p.max_logits[row] = -__builtin_inff();
    p.exp_sums[row] = 0.0f;
  }
}

// One element of a piece's normalised output: out directly when the item is
// whole, else the piece's partial row (slot = piece), written past the L2.
template <typename QT, int D>
__device__ __forceinline__ void piece_elem(const Params &p, const Work &w, int h, int d,
                                           float o) {
  const int head = w.head0 + h;
  if (!w.v2) {
    store_out_row<QT, D>(p, w.seq, head, d, o);
    return;
  }
  const size_t row = ((size_t)w.seq * p.num_heads + head) * p.max_num_partitions + w.part;
  if (p.tmp_f32)
    coherent_store_elem<float>(reinterpret_cast<float *>(p.tmp_out) + row * D + d, o);
  else
    coherent_store_elem<QT>(reinterpret_cast<QT *>(p.tmp_out) + row * D + d, o);
}

// The statistics of head h of a cut item's piece: the exp-sum l (NaN after
// an out-of-range block-table entry) and the max logit m (log2 units; stored
// in natural-log units and the absolute ALiBi convention, as wave_merge).
__device__ __forceinline__ void piece_stats(const Params &p, const Work &w, int h, float m,
                                            float l) {
  const int head = w.head0 + h;
  const size_t row = ((size_t)w.seq * p.num_heads + head) * p.max_num_partitions + w.part;
  float ml = p.alibi_slopes ? fmaf(p.alibi_slopes[head], (float)w.t_ref, m * kLn2) : m * kLn2;
  ml = l != l ? __builtin_nanf("") : ml;
  coherent_store(p.exp_sums + row, f_bits(l));
  coherent_store(p.max_logits + row, f_bits(ml));
}

// After a wave has stored its piece's partials: its arrival at the item's
// counter (lane 0, as split_merge), and in the last piece the Phase 2 merge
// of the k partials, dims across the wave's lanes.  The wavefront-scope
// fences keep the other lanes' stores before lane 0's increment and lane
// 0's result before the other lanes' loads.
template <typename QT, typename TT, int D>
__device__ __forceinline__ void piece_arrive(const Params &p, const Work &w) {
  const int lane = epi_tid() & 63;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are done
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int last = 0;
  if (lane == 0) {
    int *ctr = p.counters + (size_t)w.seq * p.num_heads + w.xslot;
    last = arrive_last(
        ctr, w.n_part,
        [](int *c) { return arrive_add(c); }, [](int *c) { arrive_acquire(c); },
        [](int *c, int v) { arrive_reset(c, v); });
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (!__builtin_amdgcn_readfirstlane(last)) return;
  // Lane c < k holds piece c's statistics, then its rescaled exp-sum r_c;
  // lanes 0 .. D/4 - 1 each merge four consecutive dims.
  const int k = min(w.n_part, kSplitMaxPieces);
  constexpr int G = D / 4;
  const TT *to = reinterpret_cast<const TT *>(p.tmp_out);
  for (int h = 0; h < w.nh; ++h) {
    const size_t row0 = ((size_t)w.seq * p.num_heads + w.head0 + h) * p.max_num_partitions;
    const float mc = lane < k ? bits_f(coherent_load(p.max_logits + row0 + lane)) : 0.0f;
    const float sc = lane < k ? bits_f(coherent_load(p.exp_sums + row0 + lane)) : 0.0f;
    float rl = 0.0f;
    const float sum = lse_rescale(
        [&](int c) { return readlane(mc, c); }, [&](int c) { return readlane(sc, c); }, k,
        [](float x) { return fast_exp2(x); }, [&](int c, float r) { rl = lane == c ? r : rl; });
    for (int g = lane; g < G; g += 64) {
      const TT *col = to + row0 * D + 4 * g;
      float o[4];
      lse_combine<4>([&](int c) { return readlane(rl, c); }, sum, k,
                     [&](int c) { return coherent_load4<TT>(col + (size_t)c * D); },
                     [](const Raw4 &r, float(&v)[4]) { unpack4<TT>(r, v); }, o);
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out_row<QT, D>(p, w.seq, w.head0 + h, 4 * g + e, o[e]);
    }
  }
}

// One element of a workgroup's result.  Wave wv left, for query head h of
// the group:
//   sm_m[wv][h]  its running max (log2 units; -inf if it saw no token)
//   sm_l[wv][h]  sum of exp2(s - m) over its tokens
//   sm_o[wv][h][d] sum of exp2(s - m) * V[d] over its tokens
// The workgroup result is the log-sum-exp combination of the four waves
// (the same rescale as the V2 page's Phase 2, applied inside one partition):
// the normalised output o, the sum and the max logit ml (natural log units).
// A NaN in sm_l (an out-of-range block-table entry) makes o and ml NaN.
template <int GS, int OSTRIDE>
__device__ __forceinline__ float wave_merge(const Params &p, const Work &w,
                                            const float (*sm_o)[GS][OSTRIDE],
                                            const float (*sm_m)[GS], const float (*sm_l)[GS],
                                            int h, int d, float &sum, float &ml) {
  float big_m = -__builtin_inff();
#pragma unroll
  for (int wv = 0; wv < kWaves; ++wv) big_m = fmaxf(big_m, sm_m[wv][h]);
  sum = 0.0f;
  float acc = 0.0f;
#pragma unroll
  for (int wv = 0; wv < kWaves; ++wv) {
    const float mw = sm_m[wv][h];
    const float c = (mw == -__builtin_inff()) ? 0.0f : fast_exp2(mw - big_m);
    sum += c * sm_l[wv][h];
    acc += c * sm_o[wv][h][d];
  }
  float o = acc / sum * p.v_scale;
  const int head = w.head0 + h;
  // The kernels add ALiBi as slope * (t - t_ref), t_ref the last token of the
  // workgroup's range (softmax inside the range is unchanged by the shift,
  // and the tokens that carry weight keep small, precise logits); the stored
  // max logit is in the absolute-position convention slope * t.
  // One rounding: the product slope * t_ref is exact inside the fma.
  ml = p.alibi_slopes ? fmaf(p.alibi_slopes[head], (float)w.t_ref, big_m * kLn2) : big_m * kLn2;
  // A wave that met an out-of-range block-table entry reports a NaN sum.
  if (sum != sum) {
    o = __builtin_nanf("");
    ml = __builtin_nanf("");
  }
  return o;
}

// Cross-wave merge and stores of a workgroup's result: out directly (v1, a
// single partition or piece), the partials of a v2 partition, or a split
// piece's partials followed by the arrival at its counter.  Must be called
// after a __syncthreads() that follows the LDS writes.
template <typename QT, int D, int GS, int OSTRIDE>
__device__ __forceinline__ void finish_partition(const Params &p, const Work &w,
                                                 const float (*sm_o)[GS][OSTRIDE],
                                                 const float (*sm_m)[GS],
                                                 const float (*sm_l)[GS]) {
  const bool split = p.mode >= kModeSplit;  // split or list: pieces merge in-kernel
  for (int idx = epi_tid(); idx < w.nh * D; idx += kThreads) {
    const int h = idx / D, d = idx - h * D;
    float sum, ml;
    const float o = wave_merge<GS, OSTRIDE>(p, w, sm_o, sm_m, sm_l, h, d, sum, ml);
    const int head = w.head0 + h;
    if (w.v2 && split) {
      const size_t row = ((size_t)w.seq * p.num_heads + head) * p.max_num_partitions + w.part;
      if (p.tmp_f32)
        coherent_store_elem<float>(reinterpret_cast<float *>(p.tmp_out) + row * D + d, o);
      else
        coherent_store_elem<QT>(reinterpret_cast<QT *>(p.tmp_out) + row * D + d, o);
      if (d == 0) {
        coherent_store(p.exp_sums + row, f_bits(sum));
        coherent_store(p.max_logits + row, f_bits(ml));
      }
    } else if (w.v2) {
      const size_t row = ((size_t)w.seq * p.num_heads + head) * p.max_num_partitions + w.part;
      if (p.tmp_f32)
        reinterpret_cast<float *>(p.tmp_out)[row * D + d] = o;
      else
        reinterpret_cast<QT *>(p.tmp_out)[row * D + d] = from_f32<QT>(o);
      if (d == 0) {
        p.exp_sums[row] = sum;
        p.max_logits[row] = ml;
      }
      if (w.single) store_out_row<QT, D>(p, w.seq, head, d, o);
    } else {
      store_out_row<QT, D>(p, w.seq, head, d, o);
    }
  }
  if (split && w.v2) {
    if (p.tmp_f32) split_merge<QT, float, D>(p, w);
    else split_merge<QT, QT, D>(p, w);
  }
}

// ---------------------------------------------------------------------------
// List mode, workgroup workers (the MFMA kernel and the VALU kernel's
// workgroup form): the epilogue of one piece, with the arrivals of cut items
// kept off the critical path.
//
// Every wave of a cut item's piece adds 1 to the item's counter, so an item
// of k pieces is complete at kWaves * k.  A piece that is not its worker's
// last stores its partials and is left pending: each of its waves arrives
// once those stores are known to be performed -- after the wave's second
// step of the worker's next item (that step's tile was requested after the
// stores, and a wave's memory operations complete in issue order), or in the
// next epilogue when it has no such step -- and when one of those arrivals
// completes the count, the workgroup merges the item in the next epilogue.
// The worker's last piece, when cut, reads the counter when it starts and,
// if at most one piece was then missing, again when it ends; once all the
// other pieces' waves have arrived it is the merger: it merges straight from
// its own result in LDS (its partials are never stored) and resets the
// counter.  Otherwise it stores its partials, drains, and thread 0 adds
// kWaves for the whole piece, the last arriver merging as in the split mode.
// ---------------------------------------------------------------------------
struct ListPend {
  int seq, xslot, head0, nh, n_part;  // the pending piece's item; n_part = 0: none pending
  bool arrived;                       // this wave has arrived for it
};

// One wave's arrival for the pending piece (lane 0's counter value before it
// in old).  Wave-uniform.
__device__ __forceinline__ void list_pend_arrive(const Params &p, ListPend &pend, int &old) {
  if (pend.n_part == 0 || pend.arrived) return;
  if ((threadIdx.x & 63) == 0)
    old = __hip_atomic_fetch_add(item_counter(p, pend.seq, pend.xslot), 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  pend.arrived = true;
}

// The epilogue.  sm_o / sm_m / sm_l hold the waves' states (written before
// an LDS barrier); final_cut: this is the worker's last piece and its item
// is cut; early: thread 0's counter reading at the piece's start; old: lane
// 0's counter value before its wave's arrival for the pending piece.  Each
// wave's memory operations up to its last step are complete (vmcnt(0)).
template <typename QT, int D, int GS, int OSTRIDE>
__device__ __forceinline__ void finish_list_piece(const Params &p, const Work &w,
                                                  float (*sm_o)[GS][OSTRIDE],
                                                  const float (*sm_m)[GS],
                                                  const float (*sm_l)[GS], ListPend &pend,
                                                  bool final_cut, int early, int old) {
  __shared__ int sm_pend_last[kWaves];
  __shared__ int sm_direct;
  __shared__ float sm_own_m[16], sm_own_s[16];
  const int tid = epi_tid(), lane = tid & 63, ew = tid >> 6;
  // The pending piece: this wave's arrival if it has not arrived yet, and
  // whether it completed the item.
  list_pend_arrive(p, pend, old);
  // (the check of wave_arrive in pa_merge.h, on the value the wave's add returned)
  if (pend.n_part && lane == 0) sm_pend_last[ew] = old == kWaves * pend.n_part - 1;
  // This piece's result: out, its partials (a pending piece), or, for a cut
  // last piece, its own rows and statistics in LDS (sm_o[0]: each element is
  // read and overwritten by the one thread that merges it).
  for (int idx = tid; idx < w.nh * D; idx += kThreads) {
    const int h = idx / D, d = idx - h * D;
    float sum, ml;
    const float o = wave_merge<GS, OSTRIDE>(p, w, sm_o, sm_m, sm_l, h, d, sum, ml);
    if (!w.v2) {
      store_out_row<QT, D>(p, w.seq, w.head0 + h, d, o);
    } else if (!final_cut) {
      const size_t row = ((size_t)w.seq * p.num_heads + w.head0 + h) * p.max_num_partitions + w.part;
      if (p.tmp_f32)
        coherent_store_elem<float>(reinterpret_cast<float *>(p.tmp_out) + row * D + d, o);
      else
        coherent_store_elem<QT>(reinterpret_cast<QT *>(p.tmp_out) + row * D + d, o);
      if (d == 0) {
        coherent_store(p.exp_sums + row, f_bits(sum));
        coherent_store(p.max_logits + row, f_bits(ml));
      }
    } else {
      sm_o[0][h][d] = o;
      if (d == 0) {
        sm_own_m[h] = ml;
        sm_own_s[h] = sum;
      }
    }
  }
  if (final_cut) {
    int *ctr = item_counter(p, w.seq, w.xslot);
    if (tid == 0) {
      int seen = early;
      if (worth_rereading(seen, w.n_part, kWaves)) seen = (int)coherent_load(ctr);
      const bool direct = others_arrived(seen, w.n_part, kWaves);
      if (direct) arrive_reset(ctr, 0);
      sm_direct = direct;
    }
    __syncthreads();
    if (sm_direct) {
      if (p.tmp_f32)
        merge_pieces<QT, float, D, OSTRIDE>(p, w.seq, w.head0, w.nh, w.n_part, w.part, sm_o[0],
                                            sm_own_m, sm_own_s);
      else
        merge_pieces<QT, QT, D, OSTRIDE>(p, w.seq, w.head0, w.nh, w.n_part, w.part, sm_o[0],
                                         sm_own_m, sm_own_s);
    } else {
      // Store the partials, then arrive for all the piece's waves at once.
      const size_t row0 = ((size_t)w.seq * p.num_heads + w.head0) * p.max_num_partitions + w.part;
      for (int idx = tid; idx < w.nh * D; idx += kThreads) {
        const int h = idx / D, d = idx - h * D;
        const size_t row = row0 + (size_t)h * p.max_num_partitions;
        if (p.tmp_f32)
          coherent_store_elem<float>(reinterpret_cast<float *>(p.tmp_out) + row * D + d, sm_o[0][h][d]);
        else
          coherent_store_elem<QT>(reinterpret_cast<QT *>(p.tmp_out) + row * D + d, sm_o[0][h][d]);
        if (d == 0) {
          coherent_store(p.exp_sums + row, f_bits(sm_own_s[h]));
          coherent_store(p.max_logits + row, f_bits(sm_own_m[h]));
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are done
      __syncthreads();
      if (tid == 0) {
        const bool last = piece_arrive_all(ctr, w.n_part, kWaves, [](int *c, int n) {
          return __hip_atomic_fetch_add(c, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        });
        if (last) arrive_reset(ctr, 0);
        sm_direct = last;
      }
      __syncthreads();
      if (sm_direct) {
        if (p.tmp_f32)
          merge_pieces<QT, float, D, 4>(p, w.seq, w.head0, w.nh, w.n_part, -1, nullptr, nullptr,
                                        nullptr);
        else
          merge_pieces<QT, QT, D, 4>(p, w.seq, w.head0, w.nh, w.n_part, -1, nullptr, nullptr,
                                     nullptr);
      }
    }
  }
  // The pending piece's item, when one of its waves' arrivals completed it.
  if (pend.n_part) {
    __syncthreads();
    const bool last = sm_pend_last[0] | sm_pend_last[1] | sm_pend_last[2] | sm_pend_last[3];
    if (last) {
      if (tid == 0) arrive_reset(item_counter(p, pend.seq, pend.xslot), 0);
      if (p.tmp_f32)
        merge_pieces<QT, float, D, 4>(p, pend.seq, pend.head0, pend.nh, pend.n_part, -1, nullptr,
                                      nullptr, nullptr);
      else
        merge_pieces<QT, QT, D, 4>(p, pend.seq, pend.head0, pend.nh, pend.n_part, -1, nullptr,
                                   nullptr, nullptr);
    }
  }
  pend.n_part = 0;
  if (w.v2 && !final_cut) {
    pend.seq = w.seq;
    pend.xslot = w.xslot;
    pend.head0 = w.head0;
    pend.nh = w.nh;
    pend.n_part = w.n_part;
    pend.arrived = false;
  }
}

}  // namespace pa
