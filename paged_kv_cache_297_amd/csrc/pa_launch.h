// Internal launcher entry points (one translation unit per element-type
// combination, so the kernel instantiations compile in parallel).  Host-side
// declarations only: this header is also compiled by a plain C++ compiler
// (the host library's sanitizer build).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/pagedattn.h"
#include "pa_params.h"

namespace pa {

enum DtCode : int { kDtF32 = 0, kDtF16 = 1, kDtBF16 = 2 };

// Where and how one kernel is launched (launch_kernel in
// pa_launch_kernel.h): with both events set, the launch records them at the
// kernel's own start and end (the profiling hook of pa_set_timing_events).
struct Launch {
  dim3 grid;
  hipStream_t stream;
  hipEvent_t start, stop;
  // Persistent (list) launch: grid.x becomes list_cus x list_per_cu workers,
  // list_per_cu = 0 meaning as many as the kernel's occupancy lets one CU
  // hold (grid.y = grid.z = 1).
  int list_cus = 0;
  int list_per_cu = 0;
  // Dynamic LDS reserved by a list launch (bytes): enough of it keeps a
  // second worker off a CU that already holds one.
  int list_lds = 0;
};

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

// Largest power-of-two head group one workgroup holds for this layout: the
// ping-pong tiles take 16 VGPRs per 1 KB load, each head 8 accumulators, 4
// query words and NL logits; wider groups are split over grid.x (their
// workgroups read the same tiles, adjacent in the grid, mostly from L2).
// Two waves per SIMD at least.
constexpr int nhd_max_group(int head_size, int block_size) {
  return head_size * block_size * 2 / 1024 >= 8 ? 2 : 4;
}

hipError_t launch_partition_valu_f32(const Params &p, int head_size, int block_size, int gp,
                                     const Launch &l);
hipError_t launch_partition_valu_f16(const Params &p, int head_size, int block_size, int gp,
                                     const Launch &l);
hipError_t launch_partition_valu_bf16(const Params &p, int head_size, int block_size, int gp,
                                      const Launch &l);
// fp8 E4M3FN cache with a 16-bit query (q_dtype kDtF16 or kDtBF16).
hipError_t launch_partition_valu_fp8(const Params &p, int q_dtype, int head_size,
                                     int block_size, int gp, const Launch &l);
hipError_t launch_partition_mfma(const Params &p, int q_dtype, bool kv_fp8, int head_size,
                                 int block_size, const Launch &l);
hipError_t launch_reduce(const Params &p, int dtype, int head_size, const Launch &l);
// Streaming read of bytes (a multiple of 16) at buf, one share per workgroup.
hipError_t launch_stream_read(const void *buf, size_t bytes, unsigned *sink, int workgroups,
                              hipStream_t stream);

// The library's own device array for paged_attention_split_static
// (PA_SPLIT_STATIC_SCRATCH_BYTES, 256-byte aligned), on the current device:
// its address, looked up once per device.
pa_status static_scratch(void **ptr);
// Zeroes n int32 words at p with a fill kernel on stream.
hipError_t launch_fill_zero(int *p, size_t n, hipStream_t stream);

// [num_blocks, Hkv, block_size, head_size] caches, 16-bit (q_dtype kDtF16 or
// kDtBF16); gp = 1, 2 or 4 query heads per workgroup (nhd_max_group).
hipError_t launch_partition_nhd(const Params &p, int q_dtype, int head_size, int block_size,
                                int gp, const Launch &l);
// MFMA partition kernel (16 query-head slots) on the same layout.
hipError_t launch_partition_mfma_rows(const Params &p, int q_dtype, int head_size,
                                      int block_size, const Launch &l);

}  // namespace pa
