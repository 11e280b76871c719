// VALU partition kernels, fp16 query and cache.
#include "pa_valu_dispatch.h"

namespace pa {
hipError_t launch_partition_valu_f16(const Params &p, int head_size, int block_size, int gp,
                                     const Launch &l) {
  return launch_valu<_Float16, _Float16>(p, head_size, block_size, gp, l);
}
}  // namespace pa
