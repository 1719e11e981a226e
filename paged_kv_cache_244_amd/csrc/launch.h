// Launch helpers shared by the host entries (pa_decode.hip, pa_prefill.hip).
// Internal to the library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "errors.h"

namespace pkv_decode {

// Dynamic LDS (bytes) that limits a launch of `fn` to `waves_per_cu`
// one-wave workgroups per compute unit; 0 when waves_per_cu <= 0.  Values below
// 4 act as 4.  Kernel and device attributes are cached.
hipError_t reserve_lds_bytes(const void* fn, int waves_per_cu, unsigned* dyn);

}  // namespace pkv_decode

namespace pkv {

// Launches `kernel` on `stream`.  When pkv_time_next_call has set events for
// the current call, the launch goes through hipExtLaunchKernel so that the
// events take the kernel's own start and end times: the call's first kernel
// records the start event, each kernel the stop event (the last one's end
// remains).  Check hipGetLastError() afterwards, as after hipLaunchKernelGGL.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, unsigned lds_bytes,
                          hipStream_t stream, Args... args) {
  CallTiming& t = call_timing();
  if (t.start || t.stop) {
    hipEvent_t start = static_cast<hipEvent_t>(t.start);
    t.start = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, start,
                          static_cast<hipEvent_t>(t.stop), 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, args...);
  }
}

}  // namespace pkv
