// Streaming read of a device buffer: the practical HBM read ceiling that the
// decode kernels' rates are compared with.  Workgroup w streams the w-th
// contiguous share of the buffer with 16-byte nontemporal loads, eight per
// thread in flight (2 KB per wave instruction group), and writes the XOR of
// the 32-bit words it read to sink[w] so that no load is dead code.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kStreamUnroll = 8;  // 16-byte loads per thread in flight

__global__ void __launch_bounds__(kThreads)
    pa_stream_read_kernel(const u32x4 *src, size_t n16, unsigned *sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t begin = per * blockIdx.x;
  const size_t end = begin + per < n16 ? begin + per : n16;
  unsigned acc = 0;
  for (size_t base = begin + threadIdx.x; base < end; base += (size_t)kThreads * kStreamUnroll) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) {
      const size_t i = base + (size_t)k * kThreads;
      v[k] = i < end ? load16_stream(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  // XOR across the workgroup: within each wave, then the four wave results.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ unsigned sm[kWaves];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = 0;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) r ^= sm[wv];
    sink[blockIdx.x] = r;
  }
}

hipError_t launch_stream_read(const void *buf, size_t bytes, unsigned *sink, int workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(pa_stream_read_kernel, dim3(workgroups), dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4 *>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pa
