// Kernel launch with optional dispatch-stamped events, for the kernels'
// launch code.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace pkv {

// Launch a kernel that takes one parameter struct.  With events, the launch
// goes through hipExtLaunchKernel, whose dispatch records them itself: they
// bracket the kernel's own execution, not the time of separate event
// records on the stream.  Returns a hipError_t as int.
template <typename P>
inline int launch_kernel(void (*kernel)(P), dim3 grid, dim3 block, void* stream, const P& p,
                         void* ev_start = nullptr, void* ev_stop = nullptr) {
  if (!ev_start && !ev_stop) {
    hipLaunchKernelGGL(kernel, grid, block, 0, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
  }
  void* args[] = {const_cast<P*>(&p)};
  return (int)hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0,
                                 static_cast<hipStream_t>(stream),
                                 static_cast<hipEvent_t>(ev_start),
                                 static_cast<hipEvent_t>(ev_stop), 0);
}

}  // namespace pkv
