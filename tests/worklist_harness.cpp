// Host emulation of the work-list decomposition of the persistent decode
// launch (paged_kv_cache_297_amd/csrc/pa_worklist.h, the arithmetic the
// kernels use): every worker's range on the line, walked item by item.
//
// stdin:  grid_workers max_seq_len window_left item_cost gx num_seqs, then the
//         num_seqs lengths.
// stdout: "T total workers W", then per worker "range w a e" (its snapped
//         range on the line) followed by one line per piece:
//         "piece w seq x start stop pieces index" (key offsets from the
//         item's 32-aligned base; stop is clipped to the item's keys).
#include <stdio.h>

#include <vector>

#include "pa_worklist.h"

int main() {
  int grid, max_len, window, item_cost, gx, b;
  if (scanf("%d %d %d %d %d %d", &grid, &max_len, &window, &item_cost, &gx, &b) != 6) return 2;
  std::vector<int> L(b), keys(b), base(b);
  std::vector<long long> cost(b), pos(b + 1, 0);
  int kmax = 0;
  for (int s = 0; s < b; ++s) {
    if (scanf("%d", &L[s]) != 1) return 2;
    keys[s] = pa::list_keys(L[s], max_len, window, &base[s]);
    cost[s] = pa::list_cost(keys[s], item_cost);
    pos[s + 1] = pos[s] + cost[s] * gx;
    kmax = keys[s] > kmax ? keys[s] : kmax;
  }
  const long long total = pos[b];
  const int workers = pa::list_workers(total, grid, kmax);
  const pa::ListShares sh = pa::list_shares(total, workers);
  printf("T %lld workers %d\n", total, workers);
  // The item holding line position t: sequence, slot, item start.
  auto locate = [&](long long t, int &s, int &x, long long &c) {
    s = 0;
    while (s + 1 < b && pos[s + 1] <= t) ++s;
    x = (int)((t - pos[s]) / cost[s]);
    if (x >= gx) x = gx - 1;
    c = pos[s] + (long long)x * cost[s];
  };
  auto snapped = [&](int w) {
    if (w >= workers) return total;
    int s, x;
    long long c;
    const long long bw = pa::list_boundary(sh, w);
    locate(bw, s, x, c);
    return c + pa::list_snap(bw - c, keys[s], cost[s]);
  };
  for (int w = 0; w < workers; ++w) {
    const long long a = snapped(w), e = snapped(w + 1);
    printf("range %d %lld %lld\n", w, a, e);
    long long t = a;
    while (t < e) {
      int s, x;
      long long c;
      locate(t, s, x, c);
      const long long start = t - c;
      const long long stop = (c + cost[s] < e ? c + cost[s] : e) - c;
      int k = 1, j = 0;
      if (keys[s] > 0) pa::list_piece(sh, c, keys[s], w, start, &k, &j);
      const long long kstop = stop < keys[s] ? stop : keys[s];
      printf("piece %d %d %d %lld %lld %d %d\n", w, s, x, start, kstop, k, j);
      t = c + cost[s];
    }
  }
  return 0;
}
