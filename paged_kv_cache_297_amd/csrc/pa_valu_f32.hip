// VALU partition kernels, fp32 query and cache.
#include "pa_valu_dispatch.h"

namespace pa {
hipError_t launch_partition_valu_f32(const Params &p, int head_size, int block_size, int gp,
                                     const Launch &l) {
  return launch_valu<float, float>(p, head_size, block_size, gp, l);
}
}  // namespace pa
