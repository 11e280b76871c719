// MFMA partition kernels: 16-bit query with a 16-bit or fp8 E4M3FN cache.
#include "pa_launch_kernel.h"
#include "pa_partition_mfma.h"

namespace pa {

// The soft cap, the sliding window and the persistent list form are
// compile-time variants.
template <typename QT, typename KVT, int D, int BS, bool LIST>
static hipError_t launch_list(const Params &p, const Launch &l) {
  const bool win = p.window_left >= 0;
  if (p.cap_on)
    return win ? launch_kernel(pa_partition_mfma<QT, KVT, D, BS, true, true, false, LIST>, l, p)
               : launch_kernel(pa_partition_mfma<QT, KVT, D, BS, true, false, false, LIST>, l, p);
  return win ? launch_kernel(pa_partition_mfma<QT, KVT, D, BS, false, true, false, LIST>, l, p)
             : launch_kernel(pa_partition_mfma<QT, KVT, D, BS, false, false, false, LIST>, l, p);
}

template <typename QT, typename KVT, int D, int BS>
static hipError_t launch_opts(const Params &p, const Launch &l) {
  return p.mode == kModeList ? launch_list<QT, KVT, D, BS, true>(p, l)
                             : launch_list<QT, KVT, D, BS, false>(p, l);
}

template <typename QT, typename KVT>
static hipError_t launch_mfma_t(const Params &p, int head_size, int block_size,
                                const Launch &l) {
#define PA_MFMA_CASE(D, BS)                                                   \
  if (head_size == D && block_size == BS) return launch_opts<QT, KVT, D, BS>(p, l);
  PA_MFMA_CASE(64, 16)
  PA_MFMA_CASE(64, 32)
  PA_MFMA_CASE(128, 16)
  PA_MFMA_CASE(128, 32)
#undef PA_MFMA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_partition_mfma(const Params &p, int q_dtype, bool kv_fp8, int head_size,
                                 int block_size, const Launch &l) {
  if (q_dtype == kDtF16)
    return kv_fp8 ? launch_mfma_t<_Float16, fp8e4m3>(p, head_size, block_size, l)
                  : launch_mfma_t<_Float16, _Float16>(p, head_size, block_size, l);
  if (q_dtype == kDtBF16)
    return kv_fp8 ? launch_mfma_t<__bf16, fp8e4m3>(p, head_size, block_size, l)
                  : launch_mfma_t<__bf16, __bf16>(p, head_size, block_size, l);
  return hipErrorInvalidValue;
}

}  // namespace pa
