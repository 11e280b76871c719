// The library-owned scratch array of paged_attention_split_static (the
// allocation-free form of paged_attention_split) and the fill kernel that
// clears its counters.
//
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy, at its own address, from the moment the code object is
// loaded until the process ends.  In host code the array's name is not a
// device address; the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that pointer is
// handed to kernels.  Calls that overlap on one GPU share the array and race.
#include <mutex>

#include "pa_launch_kernel.h"

namespace {

static __device__ __align__(256) unsigned char scratch[PA_SPLIT_STATIC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices] = {nullptr};

__global__ void __launch_bounds__(256) pa_fill_zero_kernel(int *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0;
}

}  // namespace

namespace pa {

pa_status static_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  const bool cached = dev >= 0 && dev < kMaxScratchDevices;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (cached && g_scratch_ptr[dev]) {
    *ptr = g_scratch_ptr[dev];
    return PA_OK;
  }
  void *p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
    return PA_ERR_HIP;
  if (cached) g_scratch_ptr[dev] = p;
  *ptr = p;
  return PA_OK;
}

hipError_t launch_fill_zero(int *p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  blocks = blocks < 1024 ? blocks : 1024;
  hipLaunchKernelGGL(pa_fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace pa
