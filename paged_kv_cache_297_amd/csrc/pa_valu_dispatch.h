// Maps run-time (head_size, block_size, head-group width) onto the VALU
// kernel instantiations that fit the register budget.
#pragma once

#include "pa_launch_kernel.h"
#include "pa_partition_valu.h"

namespace pa {

template <typename QT, typename KVT>
constexpr int kv_bytes_of() {
  if constexpr (sizeof(KVT) == 1) return 1;
  else return (int)sizeof(KVT);
}

template <typename QT, typename KVT, int D, int BS, int GP, int LIST>
hipError_t launch_valu_list(const Params &p, const Launch &l) {
  const bool win = p.window_left >= 0;
  if (p.cap_on)
    return win ? launch_kernel(pa_partition_valu<QT, KVT, D, BS, GP, true, true, LIST>, l, p)
               : launch_kernel(pa_partition_valu<QT, KVT, D, BS, GP, true, false, LIST>, l, p);
  return win ? launch_kernel(pa_partition_valu<QT, KVT, D, BS, GP, false, true, LIST>, l, p)
             : launch_kernel(pa_partition_valu<QT, KVT, D, BS, GP, false, false, LIST>, l, p);
}

// The soft cap, the sliding window and the persistent list form are
// compile-time variants.  The slot form (list_wave == 2) runs without a
// window only.
template <typename QT, typename KVT, int D, int BS, int GP>
hipError_t launch_valu_one(const Params &p, const Launch &l) {
  if constexpr (GP <= valu_max_group(kv_bytes_of<QT, KVT>(), D, BS)) {
    if (p.mode != kModeList) return launch_valu_list<QT, KVT, D, BS, GP, 0>(p, l);
    if (p.list_wave == 2) {
      if (p.window_left >= 0) return hipErrorInvalidValue;
      return p.cap_on ? launch_kernel(pa_partition_valu<QT, KVT, D, BS, GP, true, false, 3>, l, p)
                      : launch_kernel(pa_partition_valu<QT, KVT, D, BS, GP, false, false, 3>, l, p);
    }
    return p.list_wave ? launch_valu_list<QT, KVT, D, BS, GP, 2>(p, l)
                       : launch_valu_list<QT, KVT, D, BS, GP, 1>(p, l);
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename QT, typename KVT, int D, int BS>
hipError_t launch_valu_gp(const Params &p, int gp, const Launch &l) {
  switch (gp) {
    case 1: return launch_valu_one<QT, KVT, D, BS, 1>(p, l);
    case 2: return launch_valu_one<QT, KVT, D, BS, 2>(p, l);
    case 4: return launch_valu_one<QT, KVT, D, BS, 4>(p, l);
  }
  return hipErrorInvalidValue;
}

template <typename QT, typename KVT>
hipError_t launch_valu(const Params &p, int head_size, int block_size, int gp,
                       const Launch &l) {
  if (head_size == 64 && block_size == 16) return launch_valu_gp<QT, KVT, 64, 16>(p, gp, l);
  if (head_size == 64 && block_size == 32) return launch_valu_gp<QT, KVT, 64, 32>(p, gp, l);
  if (head_size == 128 && block_size == 16) return launch_valu_gp<QT, KVT, 128, 16>(p, gp, l);
  if (head_size == 128 && block_size == 32) return launch_valu_gp<QT, KVT, 128, 32>(p, gp, l);
  return hipErrorInvalidValue;
}

}  // namespace pa
