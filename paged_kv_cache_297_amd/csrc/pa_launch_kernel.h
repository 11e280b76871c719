// Kernel launches of the launcher translation units: plainly, or through
// hipExtLaunchKernelGGL, which records the profiling events at the kernel's
// own start and end (pa_set_timing_events).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_launch.h"

namespace pa {

// Workgroups of `kernel` (kThreads threads, static LDS only) one CU holds at
// once, from the runtime's occupancy calculator; looked up once per kernel.
inline int resident_per_cu(const void *kernel) {
  static std::mutex mu;
  static const void *keys[256];
  static int vals[256];
  static int used = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (keys[i] == kernel) return vals[i];
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0) != hipSuccess || n < 1)
    n = 1;
  if (used < 256) {
    keys[used] = kernel;
    vals[used] = n;
    ++used;
  }
  return n;
}

template <typename Kernel, typename P>
hipError_t launch_kernel(Kernel kernel, const Launch &l, const P &p) {
  dim3 grid = l.grid;
  size_t lds = 0;
  if (l.list_cus > 0) {
    const int per_cu = l.list_per_cu > 0 ? l.list_per_cu : resident_per_cu((const void *)kernel);
    grid = dim3((unsigned)(l.list_cus * per_cu), 1, 1);
    lds = (size_t)l.list_lds;
  }
  if (l.start && l.stop)
    hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), lds, l.stream, l.start, l.stop, 0, p);
  else
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), lds, l.stream, p);
  return hipGetLastError();
}

}  // namespace pa
