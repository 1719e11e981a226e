// Host-side launch planning shared by pa_decode (pa_decode.hip) and the
// host step call (allocator.cpp): which kernel serves a shape, partition and
// workspace arithmetic.  Plain C++, no HIP.  Internal to the library.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "pagedkv.h"

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

// Prefix groups (pa_decode_grouped): requests whose leading blocks are the
// same physical blocks.  blocks[i] points at request i's block ids, of which
// the first nfull[i] are full (never rewritten while shared).  Plans the
// launch as pa_decode_plan; then, if grouping saves at least
// kGroupMinSavedFraction of the batch's token reads, switches a one-pass plan
// to partitions of kGroupPartitionTokens (rounded up to the block size) and
// returns the groups ([n][PKV_GROUP_STRIDE] ints: count, members), their work
// items (group, partition) and, per request, the shared length when it ends
// inside a partition (else 0).  items holds the remaining items on return
// (plan->num_items of them); plan->workspace_bytes covers one spare partial
// slot per request.  Without a worthwhile group, groups, group_items and
// shared_lens come back empty and the plan is pa_decode_plan's.
constexpr int32_t kGroupPartitionTokens = 256;
constexpr double kGroupMinSavedFraction = 0.25;
int plan_with_groups(const int32_t* const* blocks, const int32_t* nfull, const int32_t* lens,
                     int32_t n, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t q_dtype, int32_t partition_size,
                     int32_t num_compute_units, std::vector<uint32_t>& items,
                     pkv_decode_plan* plan, std::vector<int32_t>& groups,
                     std::vector<uint32_t>& group_items, std::vector<int32_t>& shared_lens);

}  // namespace pkv_plan
