// Host-side launch planning shared by pa_decode (pa_decode.hip) and the
// host step call (allocator.cpp): which kernel serves a shape, partition and
// workspace arithmetic.  Plain C++, no HIP.  Internal to the library.
#pragma once

#include <cstddef>
#include <cstdint>

namespace pkv_plan {

// Which kernel serves this shape, and how many query heads one wave takes.
struct KernelChoice {
  bool mfma;
  int gt;
};

// MFMA kernel for fp16 queries in groups of >= 4 heads per KV head (16, 8 or 4
// heads per wave) unless the process-wide policy forces the VALU kernel (1, 2
// or 4 heads per wave).
KernelChoice choose_kernel(int32_t q_dtype, int group);

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

inline int64_t parts_for(int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || max_context_len <= 0) return 1;
  return (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
}

// Split-context workspace: unnormalised outputs [S][Hq][parts][D] and the
// (max, sum) pairs [S][Hq][parts][2], fp32, each 256-byte aligned.
inline size_t workspace_bytes_for(int32_t S, int32_t Hq, int32_t D, int64_t parts) {
  if (parts <= 1) return 0;
  const size_t n = static_cast<size_t>(S) * Hq * parts;
  return align256(n * D * sizeof(float)) + align256(n * 2 * sizeof(float));
}

// Residency limits the planner sets (waves per CU): the MFMA kernel always,
// the VALU kernel for one-pass launches over skewed lengths.
constexpr int kMfmaWavesPerCu = 6;
constexpr int kValuSkewedWavesPerCu = 4;

}  // namespace pkv_plan
