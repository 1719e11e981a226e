// Launch helpers shared by the host entries (pa_decode.hip, pa_prefill.hip).
// Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv_decode {

// Dynamic LDS (bytes) that limits a launch of `fn` to about `waves_per_cu`
// one-wave workgroups per compute unit; 0 when waves_per_cu <= 0.  Values below
// 4 act as 4.  Kernel and device attributes are cached.
hipError_t reserve_lds_bytes(const void* fn, int waves_per_cu, unsigned* dyn);

}  // namespace pkv_decode
