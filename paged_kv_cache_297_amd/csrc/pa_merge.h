// The merge of partial results and the arrival protocol of a work item cut
// into pieces, shared by the device kernels and by a host build (plain C++,
// no HIP headers) that exercises the same code on the CPU.
//
// Merge: Phase 2 of page "BI-V100 PagedAttention V2 implementation" ("Phase
// 2: Reduce across partitions (log-sum-exp)"): partials c = 0 .. k-1 with max
// logit m_c (natural-log units), exp-sum S_c and normalised output O_c give
//   M = max_c m_c,  r_c = exp(m_c - M) S_c,  out = sum_c r_c O_c / sum_c r_c.
#pragma once

#if defined(__HIPCC__)
#define PA_HD __host__ __device__
#define PA_UNROLL _Pragma("unroll")
#else
#include <math.h>
#define PA_HD
#define PA_UNROLL
#endif

namespace pa {

constexpr float kMergeLog2e = 1.4426950408889634f;

// The merge in two steps, as the kernels run it.
//
// lse_rescale, once per head: r_c = exp(m_c - M) S_c for c < k, handed to
// put_r(c, r_c) (0 for a partial with m_c = -inf, i.e., no key in its
// range); returns sum_c r_c, or NaN when some m_c is NaN (a piece that met
// an invalid block-table entry), which makes every output of the head NaN.
// m(c) = m_c, s(c) = S_c; exp2_fn(x) = 2^x.
template <typename M, typename S, typename Exp2, typename PutR>
PA_HD inline float lse_rescale(M m, S s, int k, Exp2 exp2_fn, PutR put_r) {
  const float ninf = -__builtin_inff();
  float big_m = ninf;
  bool nan_seen = false;
  for (int c = 0; c < k; ++c) {
    const float mc = m(c);
    nan_seen |= mc != mc;
    big_m = fmaxf(big_m, mc);
  }
  float sum = 0.0f;
  for (int c = 0; c < k; ++c) {
    const float mc = m(c);
    const float r = mc == ninf ? 0.0f : exp2_fn((mc - big_m) * kMergeLog2e) * s(c);
    put_r(c, r);
    sum += r;
  }
  return nan_seen ? __builtin_nanf("") : sum;
}

// Pieces whose partial rows a merge requests before it uses any of them.
constexpr int kMergeBatch = 8;

// lse_combine, per slice of N output values of one head: out[e] = sum_c
// r_c O_c[e] / sum, from r(c) = r_c and sum of lse_rescale.  load(c)
// returns piece c's slice in any raw form and unpack(raw, o) turns it into
// o[0 .. N).  A batch of kMergeBatch loads is issued, unconditionally
// (indices past k - 1 read slot k - 1 again and are not used), before any
// of them is unpacked, so their latencies overlap.  A piece with r_c = 0
// adds nothing and its slice may hold anything (an empty piece writes no
// row).  The pieces are taken in index order, so the result does not depend
// on the order in which they were produced.
template <int N, typename R, typename Load, typename Unpack>
PA_HD inline void lse_combine(R r, float sum, int k, Load load, Unpack unpack, float (&out)[N]) {
  using Raw = decltype(load(0));
  float acc[N];
  for (int e = 0; e < N; ++e) acc[e] = 0.0f;
  for (int c0 = 0; c0 < k; c0 += kMergeBatch) {
    Raw raw[kMergeBatch];
    PA_UNROLL
    for (int j = 0; j < kMergeBatch; ++j) raw[j] = load(c0 + j < k ? c0 + j : k - 1);
    PA_UNROLL
    for (int j = 0; j < kMergeBatch; ++j)
      if (c0 + j < k) {
        float o[N];
        unpack(raw[j], o);
        const float rc = r(c0 + j);
        for (int e = 0; e < N; ++e) acc[e] = rc == 0.0f ? acc[e] : fmaf(rc, o[e], acc[e]);
      }
  }
  for (int e = 0; e < N; ++e) out[e] = acc[e] / sum;
}

// The arrival of one of the k pieces of an item at the item's counter (zero
// before its first piece arrives): true for the piece that arrives last,
// which also resets the counter to zero, so the next call finds it zero.
// fetch_add(ctr) adds 1 and returns the value before the addition; its
// caller has made the piece's partial stores visible before calling it.
// acquire(ctr) runs in the last piece only, before it reads anything.
// On host threads these are a release fetch-add and an acquire load (the
// C++ memory model's form of the ordering); the device kernels pass the
// operations that give the same ordering on gfx950 (pa_partition_common.h,
// above coherent_store).  store(ctr, v) writes v.
template <typename FetchAdd, typename Acquire, typename Store>
PA_HD inline bool arrive_last(int *ctr, int k, FetchAdd fetch_add, Acquire acquire, Store store) {
  const bool last = fetch_add(ctr) == k - 1;
  if (last) {
    acquire(ctr);
    store(ctr, 0);
  }
  return last;
}

// The work list's workgroup form: every wave of a piece arrives on its own,
// so an item of k pieces is complete when the counter reaches waves * k.
// fetch_add(ctr, n) adds n and returns the value before the addition; each
// caller has made its piece's partial stores visible before arriving.
//
// A wave's arrival: true for the wave whose arrival completes the item.
template <typename FetchAdd>
PA_HD inline bool wave_arrive(int *ctr, int k, int waves, FetchAdd fetch_add) {
  return fetch_add(ctr, 1) == waves * k - 1;
}
// A worker's last piece reads the counter (seen) before it arrives: when
// every other piece's waves have arrived it is the merger, merges straight
// from its own result and never arrives (its caller resets the counter).
PA_HD inline bool others_arrived(int seen, int k, int waves) { return seen == waves * (k - 1); }
// A second read is worth its round trip when at most one piece was missing.
PA_HD inline bool worth_rereading(int seen, int k, int waves) {
  return !others_arrived(seen, k, waves) && seen >= waves * (k - 2);
}
// Otherwise the last piece stores its partials and arrives for all its
// waves at once: true when that completes the item.
template <typename FetchAdd>
PA_HD inline bool piece_arrive_all(int *ctr, int k, int waves, FetchAdd fetch_add) {
  return fetch_add(ctr, waves) == waves * (k - 1);
}

// Keys per piece when a range of len keys is cut into
// k = ceil(len / target) pieces (1 .. max_pieces) of equal length, rounded up
// to 32 keys (the MFMA step); the last piece may be shorter.
PA_HD inline int split_piece_len(int target, int len, int max_pieces) {
  int k = (len + target - 1) / target;
  k = k < max_pieces ? k : max_pieces;
  k = k > 1 ? k : 1;
  return ((len + k - 1) / k + 31) / 32 * 32;
}

}  // namespace pa
