// pa_decode entry point: argument checks, kernel choice (VALU or MFMA),
// split-context geometry and workspace, launch order.
//
// What is computed: "800 kilobytes per token" (shashforge.dev), section "The old
// answer, imported honestly", and "Only 20.4% of your KV cache held actual
// tokens" (blog.teqners.com), section "The page table, relocated into
// attention": decode attention whose kernel walks a per-request table of
// fixed-size physical blocks instead of one contiguous tensor.
//
// Kernels: pa_decode_valu.hip (one query head per wave, or any group with fp32
// queries), pa_decode_mfma.hip (groups of >= 4 query heads per KV head with fp16
// queries, on the matrix cores), pa_decode_reduce.hip (log-sum-exp combine of
// split-context partitions).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "errors.h"
#include "pa_decode_common.h"
#include "pagedkv.h"

namespace {

using pkv::fail;
using namespace pkv_decode;

constexpr float kLog2e = 1.4426950408889634f;



int head_tile(int group) {
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

// Kernel policy for head groups (see pa_decode_set_kernel_policy).  The first
// value comes from PKV_GQA_KERNEL=valu in the environment, if set.
std::atomic<int> g_policy{-1};

int kernel_policy() {
  int v = g_policy.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* env = std::getenv("PKV_GQA_KERNEL");
    const int init = (env != nullptr && std::strcmp(env, "valu") == 0) ? PKV_POLICY_VALU
                                                                       : PKV_POLICY_DEFAULT;
    g_policy.compare_exchange_strong(v, init);
    v = g_policy.load(std::memory_order_relaxed);
  }
  return v;
}

bool gqa_valu_forced() { return kernel_policy() == PKV_POLICY_VALU; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int64_t parts_for(int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || max_context_len <= 0) return 1;
  return (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
}

size_t workspace_bytes_for(int32_t S, int32_t Hq, int32_t D, int64_t parts) {
  if (parts <= 1) return 0;
  const size_t n = static_cast<size_t>(S) * Hq * parts;
  return align256(n * D * sizeof(float)) + align256(n * 2 * sizeof(float));
}

}  // namespace

extern "C" int pa_decode_set_kernel_policy(int32_t policy) {
  if (policy != PKV_POLICY_DEFAULT && policy != PKV_POLICY_VALU)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_set_kernel_policy: unknown policy %d", policy);
  const int previous = kernel_policy();
  g_policy.store(policy, std::memory_order_relaxed);
  return previous;
}

extern "C" size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                           int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return workspace_bytes_for(num_seqs, num_q_heads, head_dim,
                             parts_for(max_context_len, partition_size));
}

extern "C" int pa_decode(float* out, const void* q, int32_t q_dtype, const void* k_cache,
                         const void* v_cache, int32_t num_blocks, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         const int32_t* work_order, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, float scale, int32_t max_context_len,
                         int32_t partition_size, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq < 0 || max_context_len < 0 || partition_size < 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode: bad sizes");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_UNSUPPORTED, "pa_decode: num_q_heads %d not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (q_dtype != PKV_F32 && q_dtype != PKV_F16)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode: q_dtype %d unknown", q_dtype);
  if (partition_size % (block_size > 0 ? block_size : 1) != 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode: partition_size %d not a multiple of block_size %d",
                partition_size, block_size);
  if (num_seqs > 65535)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode: at most 65535 sequences per call");
  if (num_q_heads > 65535)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode: too many query heads");
  const int group = num_q_heads / num_kv_heads;
  const bool mfma = q_dtype == PKV_F16 && group % 4 == 0 && !gqa_valu_forced();
  const int gt = mfma ? (group % 16 == 0 ? 16 : (group % 8 == 0 ? 8 : 4)) : head_tile(group);
  KernelFn fn = mfma ? pick_mfma_kernel(head_dim, block_size, gt)
                     : pick_valu_kernel(head_dim, block_size, gt, q_dtype == PKV_F32);
  if (!fn)
    return fail(PKV_ERR_UNSUPPORTED, "pa_decode: head_dim %d / block_size %d not built", head_dim,
                block_size);
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode: NULL pointer");

  int64_t clamp64 = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  if (clamp64 > max_context_len) clamp64 = max_context_len;
  const int32_t len_clamp = static_cast<int32_t>(clamp64);
  int32_t part_tokens;
  int64_t parts;
  if (partition_size == 0) {
    const int64_t whole = (static_cast<int64_t>(len_clamp > 0 ? len_clamp : 1) + block_size - 1) /
                          block_size * block_size;
    part_tokens = static_cast<int32_t>(whole);
    parts = 1;
  } else {
    part_tokens = partition_size;
    parts = parts_for(len_clamp, partition_size);
  }
  if (parts > 65535)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode: more than 65535 partitions per request");

  DecodeParams prm{};
  prm.out = out;
  prm.q = q;
  prm.k_cache = static_cast<const uint4*>(k_cache);
  prm.v_cache = static_cast<const uint4*>(v_cache);
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.work_order = work_order;
  prm.num_seqs = num_seqs;
  prm.num_blocks = num_blocks;
  prm.max_blocks_per_seq = max_blocks_per_seq;
  prm.num_q_heads = num_q_heads;
  prm.num_kv_heads = num_kv_heads;
  prm.group = num_q_heads / num_kv_heads;
  prm.num_head_tiles = num_q_heads / gt;
  prm.scale_log2 = scale * kLog2e;
  prm.len_clamp = len_clamp;
  prm.part_tokens = part_tokens;
  prm.max_parts = static_cast<int32_t>(parts);

  if (parts > 1) {
    const size_t need = workspace_bytes_for(num_seqs, num_q_heads, head_dim, parts);
    if (!workspace || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "pa_decode: workspace of %zu bytes needed (got %zu)", need,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(PKV_ERR_WORKSPACE, "pa_decode: workspace must be 256-byte aligned");
    const size_t n = static_cast<size_t>(num_seqs) * num_q_heads * parts;
    prm.ws_o = static_cast<float*>(workspace);
    prm.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         align256(n * head_dim * sizeof(float)));
  }

  // One wave per workgroup: the dispatcher then places work at wave granularity,
  // which balances requests of unequal length across CUs far better than
  // multi-wave groups.  Grid: x = head tile (fastest), y = request in
  // work_order (longest first is the caller's best choice), z = partition.
  // Workgroups are dealt round-robin to the 8 XCDs and, inside an XCD, to its
  // shader engines, so neighbours in dispatch order must carry similar work.
  // With the partition varying fastest, a request's long first partitions and
  // short last one alternated with a fixed period and whole XCDs / shader
  // engines received only the long ones (measured: up to 2x slower on GQA).
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(prm.num_head_tiles), static_cast<unsigned>(num_seqs),
                              static_cast<unsigned>(parts)),
                     dim3(kWave), 0, st, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_decode launch: %s", hipGetErrorString(e));
  if (parts > 1) {
    e = launch_reduce(prm, head_dim, st);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_decode reduce launch: %s", hipGetErrorString(e));
  }
  return PKV_OK;
}
