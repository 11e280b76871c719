// Internal launcher entry points (one translation unit per element-type
// combination, so the kernel instantiations compile in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include "pa_params.h"

namespace pa {

enum DtCode : int { kDtF32 = 0, kDtF16 = 1, kDtBF16 = 2 };

// Largest power-of-two query-head group the VALU kernel keeps in registers
// (the query slices of one lane may use at most 64 VGPRs).
constexpr int valu_max_group(int kv_bytes, int head_size, int block_size) {
  const int loads = head_size * block_size * kv_bytes / 1024;  // 16-byte loads per tile
  const int words_per_chunk = kv_bytes == 1 ? 8 : 4;
  int g = 64 / (loads * words_per_chunk);
  if (g > 4) g = 4;
  int p2 = 1;
  while (p2 * 2 <= g) p2 *= 2;
  return p2;
}

hipError_t launch_partition_valu_f32(const Params &p, int head_size, int block_size, int gp,
                                     dim3 grid, hipStream_t stream);
hipError_t launch_partition_valu_f16(const Params &p, int head_size, int block_size, int gp,
                                     dim3 grid, hipStream_t stream);
hipError_t launch_partition_valu_bf16(const Params &p, int head_size, int block_size, int gp,
                                      dim3 grid, hipStream_t stream);
// fp8 E4M3FN cache with a 16-bit query (q_dtype kDtF16 or kDtBF16).
hipError_t launch_partition_valu_fp8(const Params &p, int q_dtype, int head_size,
                                     int block_size, int gp, dim3 grid, hipStream_t stream);
hipError_t launch_partition_mfma(const Params &p, int q_dtype, bool kv_fp8, int head_size,
                                 int block_size, dim3 grid, hipStream_t stream);
hipError_t launch_reduce(const Params &p, int dtype, int head_size, hipStream_t stream);

}  // namespace pa
