// VALU partition kernels, fp8 E4M3FN cache with an fp16 or bf16 query.
#include "pa_valu_dispatch.h"

namespace pa {
hipError_t launch_partition_valu_fp8(const Params &p, int q_dtype, int head_size,
                                     int block_size, int gp, const Launch &l) {
  if (q_dtype == kDtF16)
    return launch_valu<_Float16, fp8e4m3>(p, head_size, block_size, gp, l);
  if (q_dtype == kDtBF16)
    return launch_valu<__bf16, fp8e4m3>(p, head_size, block_size, gp, l);
  return hipErrorInvalidValue;
}
}  // namespace pa
