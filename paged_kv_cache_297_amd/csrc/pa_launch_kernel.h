// Kernel launches of the launcher translation units: plainly, or through
// hipExtLaunchKernelGGL, which records the profiling events at the kernel's
// own start and end (pa_set_timing_events).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pa_launch.h"

namespace pa {

template <typename Kernel, typename P>
hipError_t launch_kernel(Kernel kernel, const Launch &l, const P &p) {
  if (l.start && l.stop)
    hipExtLaunchKernelGGL(kernel, l.grid, dim3(kThreads), 0, l.stream, l.start, l.stop, 0, p);
  else
    hipLaunchKernelGGL(kernel, l.grid, dim3(kThreads), 0, l.stream, p);
  return hipGetLastError();
}

}  // namespace pa
