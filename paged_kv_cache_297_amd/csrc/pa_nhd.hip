// Partition kernels for the [num_blocks, Hkv, block_size, head_size] cache
// layout, 16-bit caches: the VALU form for one to four query heads per KV
// head, the MFMA form (block-rows variant) for wider groups.
#include "pa_launch_kernel.h"
#include "pa_partition_mfma.h"
#include "pa_partition_nhd.h"

namespace pa {

template <typename QT, int D, int BS, int GP>
static hipError_t launch_nhd_opts(const Params &p, const Launch &l) {
  if constexpr (GP <= nhd_max_group(D, BS)) {
    const bool win = p.window_left >= 0;
    if (p.cap_on)
      return win ? launch_kernel(pa_partition_nhd<QT, D, BS, GP, true, true>, l, p)
                 : launch_kernel(pa_partition_nhd<QT, D, BS, GP, true, false>, l, p);
    return win ? launch_kernel(pa_partition_nhd<QT, D, BS, GP, false, true>, l, p)
               : launch_kernel(pa_partition_nhd<QT, D, BS, GP, false, false>, l, p);
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename QT, int D, int BS>
static hipError_t launch_nhd_gp(const Params &p, int gp, const Launch &l) {
  switch (gp) {
    case 1: return launch_nhd_opts<QT, D, BS, 1>(p, l);
    case 2: return launch_nhd_opts<QT, D, BS, 2>(p, l);
    case 4: return launch_nhd_opts<QT, D, BS, 4>(p, l);
  }
  return hipErrorInvalidValue;
}

template <typename QT>
static hipError_t launch_nhd_t(const Params &p, int head_size, int block_size, int gp,
                               const Launch &l) {
  if (head_size == 64 && block_size == 16) return launch_nhd_gp<QT, 64, 16>(p, gp, l);
  if (head_size == 64 && block_size == 32) return launch_nhd_gp<QT, 64, 32>(p, gp, l);
  if (head_size == 128 && block_size == 16) return launch_nhd_gp<QT, 128, 16>(p, gp, l);
  if (head_size == 128 && block_size == 32) return launch_nhd_gp<QT, 128, 32>(p, gp, l);
  return hipErrorInvalidValue;
}

hipError_t launch_partition_nhd(const Params &p, int q_dtype, int head_size, int block_size,
                                int gp, const Launch &l) {
  if (q_dtype == kDtF16) return launch_nhd_t<_Float16>(p, head_size, block_size, gp, l);
  if (q_dtype == kDtBF16) return launch_nhd_t<__bf16>(p, head_size, block_size, gp, l);
  return hipErrorInvalidValue;
}

// The soft cap, the sliding window and the persistent list form are
// compile-time variants.
template <typename QT, int D, int BS, bool LIST>
static hipError_t launch_rows_mfma_list(const Params &p, const Launch &l) {
  const bool win = p.window_left >= 0;
  if (p.cap_on)
    return win ? launch_kernel(pa_partition_mfma<QT, QT, D, BS, true, true, true, LIST>, l, p)
               : launch_kernel(pa_partition_mfma<QT, QT, D, BS, true, false, true, LIST>, l, p);
  return win ? launch_kernel(pa_partition_mfma<QT, QT, D, BS, false, true, true, LIST>, l, p)
             : launch_kernel(pa_partition_mfma<QT, QT, D, BS, false, false, true, LIST>, l, p);
}

template <typename QT, int D, int BS>
static hipError_t launch_rows_mfma_opts(const Params &p, const Launch &l) {
  return p.mode == kModeList ? launch_rows_mfma_list<QT, D, BS, true>(p, l)
                             : launch_rows_mfma_list<QT, D, BS, false>(p, l);
}

template <typename QT>
static hipError_t launch_rows_mfma_t(const Params &p, int head_size, int block_size,
                                     const Launch &l) {
  if (head_size == 64 && block_size == 16) return launch_rows_mfma_opts<QT, 64, 16>(p, l);
  if (head_size == 64 && block_size == 32) return launch_rows_mfma_opts<QT, 64, 32>(p, l);
  if (head_size == 128 && block_size == 16) return launch_rows_mfma_opts<QT, 128, 16>(p, l);
  if (head_size == 128 && block_size == 32) return launch_rows_mfma_opts<QT, 128, 32>(p, l);
  return hipErrorInvalidValue;
}

hipError_t launch_partition_mfma_rows(const Params &p, int q_dtype, int head_size,
                                      int block_size, const Launch &l) {
  if (q_dtype == kDtF16) return launch_rows_mfma_t<_Float16>(p, head_size, block_size, l);
  if (q_dtype == kDtBF16) return launch_rows_mfma_t<__bf16>(p, head_size, block_size, l);
  return hipErrorInvalidValue;
}

}  // namespace pa
