// pkv_check_tables: a debug pass over device-resident block tables, off the
// decode path.  "The KV cache is a systems problem" (rsw.lol), section "Shared
// prefixes need ownership rules": a review of a paged cache follows each
// physical block through its lifecycle, and stale or foreign ids in a table
// handed to the GPU are the symptom of a lifecycle mistake.  The decode and
// prefill kernels skip ids outside the pool so that bad input cannot fault;
// this pass makes such input visible instead of silently skipped.
//
// One workgroup walks every request: its length must be >= 0 and its context
// must fit its table row, and every entry that covers the context must name a
// block of the pool.  The counts and the first offender are reduced in LDS and
// written by one thread, so the result needs no atomics and no zeroed buffer.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "errors.h"
#include "launch.h"
#include "pagedkv.h"

namespace {

using pkv::fail;

constexpr int kCheckThreads = 1024;
constexpr int64_t kNoOffender = INT64_MAX;

// Offender key: ordered by request, then by block index, a length error (block
// index -1) first; bit layout request << 33 | (block index + 1).
__device__ __forceinline__ int64_t offender_key(int32_t seq, int32_t block) {
  return (static_cast<int64_t>(seq) << 33) | static_cast<int64_t>(block + 1);
}

__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(
    const int32_t* __restrict__ tables, int32_t max_blocks, const int32_t* __restrict__ lens,
    int32_t num_seqs, int32_t block_size, int32_t num_blocks, int32_t* __restrict__ result) {
  __shared__ int32_t s_bad[kCheckThreads];
  __shared__ int32_t s_len[kCheckThreads];
  __shared__ int64_t s_first[kCheckThreads];
  const int t = threadIdx.x;
  int32_t bad = 0, bad_len = 0;
  int64_t first = kNoOffender;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t len = lens[s];
    const int64_t need = len < 0 ? 0 : (static_cast<int64_t>(len) + block_size - 1) / block_size;
    if (len < 0 || need > max_blocks) {
      if (t == 0) {
        ++bad_len;
        first = first < offender_key(s, -1) ? first : offender_key(s, -1);
      }
    }
    const int32_t n = static_cast<int32_t>(need < max_blocks ? need : max_blocks);
    const int32_t* row = tables + static_cast<int64_t>(s) * max_blocks;
    for (int32_t j = t; j < n; j += kCheckThreads) {
      const int32_t id = row[j];
      if (id < 0 || id >= num_blocks) {
        ++bad;
        const int64_t k = offender_key(s, j);
        first = first < k ? first : k;
      }
    }
  }
  s_bad[t] = bad;
  s_len[t] = bad_len;
  s_first[t] = first;
  __syncthreads();
  for (int w = kCheckThreads / 2; w > 0; w >>= 1) {
    if (t < w) {
      s_bad[t] += s_bad[t + w];
      s_len[t] += s_len[t + w];
      s_first[t] = s_first[t] < s_first[t + w] ? s_first[t] : s_first[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    const int64_t f = s_first[0];
    result[0] = s_bad[0];
    result[1] = s_len[0];
    result[2] = f == kNoOffender ? -1 : static_cast<int32_t>(f >> 33);
    result[3] = f == kNoOffender ? -1 : static_cast<int32_t>((f & ((int64_t{1} << 33) - 1)) - 1);
  }
}

}  // namespace

extern "C" int pkv_check_tables(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                                int32_t num_blocks, int32_t* result, void* stream) {
  if (num_seqs < 0 || num_seqs > (1 << 30) || max_blocks_per_seq < 0 || block_size <= 0 ||
      num_blocks < 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_check_tables: bad sizes");
  if (!result) return fail(PKV_ERR_INVALID_ARG, "pkv_check_tables: NULL result");
  if (num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !block_tables)))
    return fail(PKV_ERR_INVALID_ARG, "pkv_check_tables: NULL tables or lengths");
  pkv::launch_kernel(check_tables_kernel, dim3(1), dim3(kCheckThreads), 0,
                     static_cast<hipStream_t>(stream), block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, block_size, num_blocks, result);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_check_tables launch: %s", hipGetErrorString(e));
  return PKV_OK;
}
