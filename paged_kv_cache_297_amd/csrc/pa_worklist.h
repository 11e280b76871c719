// Work-list decomposition of a decode batch for the persistent launch
// (paged_attention_worklist), shared by the device kernels and by a host
// build (plain C++) that checks it on the CPU.
//
// Items.  Item (s, x) is sequence s with grid-x slot x (KV head x query-head
// group), x = 0 .. gx-1, in sequence-major order.  Its keys run from the
// 32-aligned start of its window, base_s, to its length L_s.  Its cost is the
// memory-load model of the PoD page (FlashInfer PR #967, the work estimate
// qo_len + 2 * page_size * kv_len, which its author describes as modelling
// memory load rather than compute): a per-request term plus two rows (K and
// V) per key, i.e., in units of a key's K and V rows, cost = keys + item_cost.
// item_cost is the per-item term (the library calibrates it to an item's
// fixed cost); an empty or invalid sequence costs 1 + item_cost, so its
// output still has an owner.
//
// Line.  The items lie end to end on a line of total length T = gx * sum_s
// cost_s, item (s, x) at C = gx * P_s + x * cost_s with P_s the cost of the
// sequences before s.  Worker w of W takes [snap(b_w), snap(b_{w+1})) with
// b_w = floor(w * T / W).  snap() moves a position that falls inside an item
// within kListMinPiece keys of either end to that end, and otherwise down to
// a multiple of kListStep keys from the item's base: every piece of a cut
// item spans at least kListMinPiece keys (so an item of L keys has at most
// L / 512 pieces, which fit its partition slots), and every cut falls on a
// 32-key step.  Workers with a range of at least kListMinRange keys never
// see an empty range.
#pragma once

#if defined(__HIPCC__)
#define PA_LHD __host__ __device__
#else
#define PA_LHD
#endif

namespace pa {

constexpr int kListMinPiece = 512;   // keys: shortest piece of a cut item
constexpr int kListStep = 32;        // keys: cuts fall on these steps from the item's base
constexpr int kListMinRange = 2048;  // keys: shortest range of a worker
constexpr int kListMaxPieces = 64;   // pieces of one item (the merge keeps their statistics in LDS)
constexpr int kListMaxWorkers = 65535;  // workers of one launch (keeps list_boundary in 32 bits)

// Keys of a sequence of length L for the list (0 when empty or invalid) and
// the 32-aligned first key `base` the key offsets count from.
PA_LHD inline int list_keys(int L, int max_seq_len, int window_left, int *base) {
  *base = 0;
  if (L <= 0 || L > max_seq_len) return 0;
  const int t_lo = (window_left >= 0 && L - 1 - window_left > 0) ? L - 1 - window_left : 0;
  *base = t_lo / kListStep * kListStep;
  return L - *base;
}

PA_LHD inline long long list_cost(int keys, int item_cost) {
  return (long long)(keys > 1 ? keys : 1) + item_cost;
}

// floor(a / b) for 0 <= a < 2^62, 1 <= b < 2^31, exactly: a double quotient
// corrected by integer products.
PA_LHD inline long long list_div(long long a, long long b) {
  long long q = (long long)((double)a / (double)b);
  while (q > 0 && q * b > a) --q;
  while ((q + 1) * b <= a) ++q;
  return q;
}

// Workers that get work: at most W (and kListMaxWorkers), and few enough
// that each range spans at least max(kListMinRange, max_keys /
// (kListMaxPieces - 2)) keys, so that no range is empty and no item is cut
// into more than kListMaxPieces pieces.
PA_LHD inline int list_workers(long long total, int grid_workers, int max_keys) {
  long long r = (max_keys + kListMaxPieces - 3) / (kListMaxPieces - 2);
  r = r > kListMinRange ? r : kListMinRange;
  long long w = list_div(total, r);
  w = w < grid_workers ? w : grid_workers;
  w = w < kListMaxWorkers ? w : kListMaxWorkers;
  return (int)(w < 1 ? 1 : w);
}

// The line cut into W equal shares: b_w = floor(w * T / W) = w q + floor(w r
// / W) with T = q W + r, without overflow (w <= W).
struct ListShares {
  long long total, q, r;
  int workers;
};

PA_LHD inline ListShares list_shares(long long total, int workers) {
  ListShares sh;
  sh.total = total;
  sh.workers = workers;
  sh.q = list_div(total, workers);
  sh.r = total - sh.q * workers;
  return sh;
}

// w r < W^2 < 2^32 (list_workers keeps W below 2^16), so the remainder
// term is one 32-bit division.
PA_LHD inline long long list_boundary(const ListShares &sh, int w) {
  return (long long)w * sh.q +
         (long long)((unsigned)((long long)w * sh.r) / (unsigned)sh.workers);
}

// A position at key offset o of an item (0 <= o < cost) snapped as described
// above; returns the snapped offset, `cost` standing for the item's end.
PA_LHD inline long long list_snap(long long o, int keys, long long cost) {
  if (o < kListMinPiece) return 0;
  if (keys - o < kListMinPiece) return cost;
  return o / kListStep * kListStep;
}

// Smallest w in [lo, hi] with b_w >= x (hi + 1 if none).  b_w >= x exactly
// when w >= x W / T, so the answer is ceil(x W / T) clamped to the range: a
// double estimate, corrected by stepping while the boundaries say so.
PA_LHD inline int list_first_at_or_after(const ListShares &sh, long long x, int lo, int hi) {
  long long v = x <= 0 ? 0 : (long long)((double)x * (double)sh.workers / (double)sh.total);
  v = v < lo ? lo : (v > hi + 1 ? hi + 1 : v);
  while (v > lo && list_boundary(sh, (int)v - 1) >= x) --v;
  while (v <= hi && list_boundary(sh, (int)v) < x) ++v;
  return (int)v;
}

// Pieces of the item at line position c with `keys` keys, and the index of
// the piece that worker w starts at key offset `start` (0 when the piece
// starts at the item's start).  The cuts inside the item are the boundaries
// b_v (1 <= v <= W-1) with c + 512 <= b_v <= c + keys - 512; they are taken
// in order, so piece j starts at the j-th of them.
PA_LHD inline void list_piece(const ListShares &sh, long long c, int keys, int w,
                              long long start, int *pieces, int *index) {
  *pieces = 1;
  *index = 0;
  if (keys < 2 * kListMinPiece || sh.workers < 2) return;
  const int va = list_first_at_or_after(sh, c + kListMinPiece, 1, sh.workers - 1);
  const int vb = list_first_at_or_after(sh, c + keys - kListMinPiece + 1, 1, sh.workers - 1) - 1;
  *pieces = vb >= va ? vb - va + 2 : 1;
  *index = start > 0 ? w - va + 1 : 0;
}

}  // namespace pa
