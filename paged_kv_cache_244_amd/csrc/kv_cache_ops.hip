// Slot-mapped K/V write and copy-on-write block copy for the paged KV cache.
//
// kv_cache_write: "Only 20.4% of your KV cache held actual tokens"
// (blog.teqners.com), section "The page table, relocated into attention" — each
// new token lands in the next slot of its request's last logical block, which
// lives in some physical block of the pool.
// kv_copy_blocks: same page, section "The part everyone forgets: pages enable
// sharing, not just packing" — a write into a shared, partly filled block is
// preceded by copying one whole block into a fresh one.
//
// Both are bit copies of fp16 data moved as 16-byte vectors; they are bound by
// HBM bandwidth (2 bytes moved per byte copied), not by arithmetic.
//
// pkv_upload: the per-step host data (slots, copy pairs, block tables, lengths,
// work items) read by a kernel straight from pinned host memory and stored in
// device memory, on the caller's stream.  Same page, section "The page table,
// relocated into attention": the tables are made on the host and must be in
// GPU memory before the kernel walks them.  pkv_upload_write does that copy and
// the step's kv_cache_write in one launch.
// kv_swap_blocks: "The KV cache is a systems problem" (rsw.lol), section
// "Eviction and reuse can move costs elsewhere" — evicted blocks moved to a
// pool in pinned host memory and back, block by block, by the same copy kernel
// as copy-on-write: the host pool is addressed over the bus, so both
// directions run on the caller's compute stream without a copy-engine hand-off,
// bound by the host link rather than by HBM.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "errors.h"
#include "launch.h"
#include "pagedkv.h"

namespace {

using pkv::fail;

constexpr int kThreads = 256;

bool supported_geometry(int32_t head_dim, int32_t block_size) {
  bool d_ok = head_dim == 64 || head_dim == 128;
  bool b_ok = block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64 ||
              block_size == 128;
  return d_ok && b_ok;
}

// One thread moves one 16-byte chunk (8 halves) of one token's K and V.
// chunk index = token * chunks_per_token + head * chunks_per_row + d8.  Workgroup
// `wg` of `nwg` takes chunks wg * kThreads + lane, then every nwg * kThreads.
__device__ __forceinline__ void write_chunks(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, const uint4* __restrict__ k_new,
    const uint4* __restrict__ v_new, const int64_t* __restrict__ slot_mapping, int64_t total_chunks,
    int32_t chunks_per_token, int32_t chunks_per_row, int32_t block_size, int64_t num_slots,
    int64_t wg, int64_t nwg) {
  const int64_t stride = nwg * kThreads;
  for (int64_t idx = wg * kThreads + threadIdx.x; idx < total_chunks; idx += stride) {
    const int64_t token = idx / chunks_per_token;
    const int32_t c = static_cast<int32_t>(idx - token * chunks_per_token);
    const int64_t slot = slot_mapping[token];
    if (slot < 0 || slot >= num_slots) continue;   // skip marker / guard against bad slots
    const int64_t block = slot / block_size;
    const int32_t offset = static_cast<int32_t>(slot - block * block_size);
    const int32_t head = c / chunks_per_row;
    const int32_t d8 = c - head * chunks_per_row;
    // [block][head][offset][d8] in 16-byte units; chunks_per_token = heads * chunks_per_row.
    const int64_t dst =
        ((block * (chunks_per_token / chunks_per_row) + head) * block_size + offset) * chunks_per_row + d8;
    k_cache[dst] = k_new[idx];
    v_cache[dst] = v_new[idx];
  }
}

__global__ __launch_bounds__(kThreads) void kv_cache_write_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, const uint4* __restrict__ k_new,
    const uint4* __restrict__ v_new, const int64_t* __restrict__ slot_mapping, int64_t total_chunks,
    int32_t chunks_per_token, int32_t chunks_per_row, int32_t block_size, int64_t num_slots) {
  write_chunks(k_cache, v_cache, k_new, v_new, slot_mapping, total_chunks, chunks_per_token,
               chunks_per_row, block_size, num_slots, blockIdx.x, gridDim.x);
}

// Host-to-device copy as a kernel: 16 bytes per lane, grid-stride.  The loads
// cross PCIe (the source is pinned host memory the GPU can address); running
// on the compute queue keeps the step's kernels free of copy-engine handoffs.
__device__ __forceinline__ void copy16(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                       int64_t n16, int64_t wg, int64_t nwg) {
  const int64_t stride = nwg * kThreads;
  for (int64_t i = wg * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void upload_kernel(uint4* __restrict__ dst,
                                                          const uint4* __restrict__ src,
                                                          int64_t n16) {
  copy16(dst, src, n16, blockIdx.x, gridDim.x);
}

// The upload and the write of a decode step in one launch: workgroups
// [0, up_wgs) copy the step buffer, the rest write the new tokens, reading their
// slots from the pinned buffer itself (its device copy is being made by this
// same launch).  One launch instead of two saves a kernel boundary per step.
__global__ __launch_bounds__(kThreads) void upload_write_kernel(
    uint4* __restrict__ dst, const uint4* __restrict__ src, int64_t n16, int32_t up_wgs,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, const uint4* __restrict__ k_new,
    const uint4* __restrict__ v_new, const int64_t* __restrict__ slot_mapping, int64_t total_chunks,
    int32_t chunks_per_token, int32_t chunks_per_row, int32_t block_size, int64_t num_slots) {
  if (static_cast<int32_t>(blockIdx.x) < up_wgs) {
    copy16(dst, src, n16, blockIdx.x, up_wgs);
  } else {
    write_chunks(k_cache, v_cache, k_new, v_new, slot_mapping, total_chunks, chunks_per_token,
                 chunks_per_row, block_size, num_slots, blockIdx.x - up_wgs, gridDim.x - up_wgs);
  }
}

constexpr int kMaxLayersPerLaunch = 32;

// Source and destination pools of each layer: the same pools for copy-on-write,
// a device pool and a pinned host pool (device-side addresses) for a swap.
struct LayerPools {
  const uint4* src_k[kMaxLayersPerLaunch];
  const uint4* src_v[kMaxLayersPerLaunch];
  uint4* dst_k[kMaxLayersPerLaunch];
  uint4* dst_v[kMaxLayersPerLaunch];
};

constexpr int kCopyUnroll = 4;

// grid: x = chunk groups within one block, y = pair, z = layer * 2 + (0: K, 1: V).
// A block is contiguous: heads * block_size * head_dim halves = chunks_per_block
// 16-byte chunks.  Each thread issues kCopyUnroll loads before its stores.
__global__ __launch_bounds__(kThreads) void kv_copy_blocks_kernel(
    LayerPools pools, const int32_t* __restrict__ pairs, int32_t src_blocks, int32_t dst_blocks,
    int64_t chunks_per_block) {
  const int32_t src = pairs[2 * blockIdx.y];
  const int32_t dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const int layer = blockIdx.z >> 1;
  const uint4* s = ((blockIdx.z & 1) ? pools.src_v[layer] : pools.src_k[layer]) +
                   static_cast<int64_t>(src) * chunks_per_block;
  uint4* d = ((blockIdx.z & 1) ? pools.dst_v[layer] : pools.dst_k[layer]) +
             static_cast<int64_t>(dst) * chunks_per_block;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kThreads * kCopyUnroll + threadIdx.x;
  uint4 tmp[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = first + u * kThreads;
    if (i < chunks_per_block) tmp[u] = s[i];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = first + u * kThreads;
    if (i < chunks_per_block) d[i] = tmp[u];
  }
}

int hip_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

// The address a kernel uses for `p`, which must be device memory or pinned host
// memory (the runtime knows both; anything else, e.g. pageable host memory, is
// refused, since a kernel touching it would fault).  nullptr on refusal.
const void* kernel_address(const void* p, bool* is_host) {
  hipPointerAttribute_t at{};
  if (p == nullptr || hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (at.type == hipMemoryTypeDevice) {
    *is_host = false;
    return p;
  }
  if (at.type != hipMemoryTypeHost || at.devicePointer == nullptr) return nullptr;
  *is_host = true;
  const char* dev = static_cast<const char*>(at.devicePointer);
  if (at.hostPointer != nullptr && at.hostPointer != p)   // attributes of the allocation base
    dev += static_cast<const char*>(p) - static_cast<const char*>(at.hostPointer);
  return dev;
}

// Launches the block copy for every layer, kMaxLayersPerLaunch layers at a time.
int launch_block_copy(const void* const* src_k, const void* const* src_v, void* const* dst_k,
                      void* const* dst_v, int32_t num_layers, const int32_t* block_pairs,
                      int32_t num_pairs, int32_t src_blocks, int32_t dst_blocks,
                      int64_t chunks_per_block, bool translate, hipStream_t stream,
                      const char* what) {
  const int64_t per_wg = static_cast<int64_t>(kThreads) * kCopyUnroll;
  const unsigned gx = static_cast<unsigned>((chunks_per_block + per_wg - 1) / per_wg);
  for (int32_t first = 0; first < num_layers; first += kMaxLayersPerLaunch) {
    const int32_t n = num_layers - first < kMaxLayersPerLaunch ? num_layers - first
                                                               : kMaxLayersPerLaunch;
    LayerPools pools{};
    for (int32_t l = 0; l < n; ++l) {
      const void* sk = src_k[first + l];
      const void* sv = src_v[first + l];
      void* dk = dst_k[first + l];
      void* dv = dst_v[first + l];
      if (!sk || !sv || !dk || !dv)
        return fail(PKV_ERR_INVALID_ARG, "%s: NULL pool for layer %d", what, first + l);
      if (translate) {
        bool host[4];
        sk = kernel_address(sk, &host[0]);
        sv = kernel_address(sv, &host[1]);
        dk = const_cast<void*>(kernel_address(dk, &host[2]));
        dv = const_cast<void*>(kernel_address(dv, &host[3]));
        if (!sk || !sv || !dk || !dv)
          return fail(PKV_ERR_INVALID_ARG,
                      "%s: a pool of layer %d is neither device memory nor pinned host memory",
                      what, first + l);
      }
      if ((reinterpret_cast<uintptr_t>(sk) | reinterpret_cast<uintptr_t>(sv) |
           reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv)) % 16 != 0)
        return fail(PKV_ERR_INVALID_ARG, "%s: pools must be 16-byte aligned", what);
      pools.src_k[l] = static_cast<const uint4*>(sk);
      pools.src_v[l] = static_cast<const uint4*>(sv);
      pools.dst_k[l] = static_cast<uint4*>(dk);
      pools.dst_v[l] = static_cast<uint4*>(dv);
    }
    pkv::launch_kernel(kv_copy_blocks_kernel, dim3(gx, num_pairs, 2 * n), dim3(kThreads), 0,
                       stream, pools, block_pairs, src_blocks, dst_blocks, chunks_per_block);
    if (int rc = hip_status(what)) return rc;
  }
  return PKV_OK;
}

}  // namespace

extern "C" int kv_cache_write(void* k_cache, void* v_cache, int32_t num_blocks, const void* k_new,
                              const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_write: bad sizes (tokens %d, blocks %d, heads %d)",
                num_tokens, num_blocks, num_kv_heads);
  if (!supported_geometry(head_dim, block_size))
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write: head_dim %d / block_size %d not built",
                head_dim, block_size);
  if (num_tokens == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "kv_cache_write: NULL pointer");
  const int32_t chunks_per_row = head_dim / 8;
  const int32_t chunks_per_token = num_kv_heads * chunks_per_row;
  const int64_t total = static_cast<int64_t>(num_tokens) * chunks_per_token;
  const int64_t want_blocks = (total + kThreads - 1) / kThreads;
  const unsigned grid = static_cast<unsigned>(want_blocks < 65536 * 16 ? want_blocks : 65536 * 16);
  pkv::launch_kernel(kv_cache_write_kernel, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), static_cast<const uint4*>(k_new),
                     static_cast<const uint4*>(v_new), slot_mapping, total, chunks_per_token,
                     chunks_per_row, block_size, static_cast<int64_t>(num_blocks) * block_size);
  return hip_status("kv_cache_write launch");
}

extern "C" int kv_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              const int32_t* block_pairs, int32_t num_pairs, int32_t num_blocks,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  if (num_layers < 0 || num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID_ARG, "kv_copy_blocks: bad sizes");
  if (!supported_geometry(head_dim, block_size))
    return fail(PKV_ERR_UNSUPPORTED, "kv_copy_blocks: head_dim %d / block_size %d not built",
                head_dim, block_size);
  if (num_pairs == 0 || num_layers == 0) return PKV_OK;
  if (!k_caches || !v_caches || !block_pairs)
    return fail(PKV_ERR_INVALID_ARG, "kv_copy_blocks: NULL pointer");
  if (num_pairs > 65535)
    return fail(PKV_ERR_INVALID_ARG, "kv_copy_blocks: at most 65535 pairs per call (got %d)",
                num_pairs);
  const int64_t chunks_per_block = static_cast<int64_t>(num_kv_heads) * block_size * head_dim / 8;
  return launch_block_copy(k_caches, v_caches, k_caches, v_caches, num_layers, block_pairs,
                           num_pairs, num_blocks, num_blocks, chunks_per_block, false,
                           static_cast<hipStream_t>(stream), "kv_copy_blocks launch");
}

extern "C" int kv_swap_blocks(void* const* dst_k, void* const* dst_v, int32_t dst_num_blocks,
                              void* const* src_k, void* const* src_v, int32_t src_num_blocks,
                              int32_t num_layers, const int32_t* block_pairs, int32_t num_pairs,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  if (num_layers < 0 || num_pairs < 0 || dst_num_blocks <= 0 || src_num_blocks <= 0 ||
      num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID_ARG, "kv_swap_blocks: bad sizes");
  if (!supported_geometry(head_dim, block_size))
    return fail(PKV_ERR_UNSUPPORTED, "kv_swap_blocks: head_dim %d / block_size %d not built",
                head_dim, block_size);
  if (num_pairs == 0 || num_layers == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !block_pairs)
    return fail(PKV_ERR_INVALID_ARG, "kv_swap_blocks: NULL pointer");
  if (num_pairs > 65535)
    return fail(PKV_ERR_INVALID_ARG, "kv_swap_blocks: at most 65535 pairs per call (got %d)",
                num_pairs);
  const int64_t chunks_per_block = static_cast<int64_t>(num_kv_heads) * block_size * head_dim / 8;
  return launch_block_copy(src_k, src_v, dst_k, dst_v, num_layers, block_pairs, num_pairs,
                           src_num_blocks,
                           dst_num_blocks, chunks_per_block, true,
                           static_cast<hipStream_t>(stream), "kv_swap_blocks launch");
}

extern "C" int pkv_upload(void* dst, const void* src, uint64_t bytes, void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  if (bytes == 0) return PKV_OK;
  if (!dst || !src) return fail(PKV_ERR_INVALID_ARG, "pkv_upload: NULL pointer");
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_upload: pointers and size must be multiples of 16");
  // The kernel may only touch memory the GPU can address: the source must be
  // pinned host memory and the destination device memory.  Anything else is
  // refused before a launch.
  bool src_host = false, dst_host = true;
  const char* dev_src = static_cast<const char*>(kernel_address(src, &src_host));
  if (!dev_src || !src_host)
    return fail(PKV_ERR_INVALID_ARG, "pkv_upload: source is not pinned host memory");
  if (!kernel_address(dst, &dst_host) || dst_host)
    return fail(PKV_ERR_INVALID_ARG, "pkv_upload: destination is not device memory");
  if (reinterpret_cast<uintptr_t>(dev_src) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_upload: device address of the source is misaligned");
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  int64_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;
  pkv::launch_kernel(upload_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(dst),
                     reinterpret_cast<const uint4*>(dev_src), n16);
  return hip_status("pkv_upload launch");
}

extern "C" int pkv_upload_write(void* dst, const void* src, uint64_t bytes, void* k_cache,
                                void* v_cache, int32_t num_blocks, const void* k_new,
                                const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_upload_write: bad sizes (tokens %d, blocks %d, heads %d)",
                num_tokens, num_blocks, num_kv_heads);
  if (!supported_geometry(head_dim, block_size))
    return fail(PKV_ERR_UNSUPPORTED, "pkv_upload_write: head_dim %d / block_size %d not built",
                head_dim, block_size);
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_upload_write: pointers and size must be multiples of 16");
  if (bytes == 0 && num_tokens == 0) return PKV_OK;
  const char* dev_src = nullptr;
  if (bytes > 0) {
    if (!dst || !src) return fail(PKV_ERR_INVALID_ARG, "pkv_upload_write: NULL buffer");
    bool src_host = false, dst_host = true;
    dev_src = static_cast<const char*>(kernel_address(src, &src_host));
    if (!dev_src || !src_host)
      return fail(PKV_ERR_INVALID_ARG, "pkv_upload_write: source is not pinned host memory");
    if (!kernel_address(dst, &dst_host) || dst_host)
      return fail(PKV_ERR_INVALID_ARG, "pkv_upload_write: destination is not device memory");
    if (reinterpret_cast<uintptr_t>(dev_src) % 16 != 0)
      return fail(PKV_ERR_INVALID_ARG, "pkv_upload_write: device address of the source is misaligned");
  }
  const int64_t* dev_slots = nullptr;
  if (num_tokens > 0) {
    if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
      return fail(PKV_ERR_INVALID_ARG, "pkv_upload_write: NULL pointer");
    bool slots_host = false;
    dev_slots = static_cast<const int64_t*>(kernel_address(slot_mapping, &slots_host));
    if (!dev_slots)
      return fail(PKV_ERR_INVALID_ARG,
                  "pkv_upload_write: slot_mapping is neither device memory nor pinned host memory");
  }
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  int64_t up = (n16 + kThreads - 1) / kThreads;
  if (up > 1024) up = 1024;
  const int32_t chunks_per_row = head_dim / 8;
  const int32_t chunks_per_token = num_kv_heads * chunks_per_row;
  const int64_t total = static_cast<int64_t>(num_tokens) * chunks_per_token;
  int64_t wr = (total + kThreads - 1) / kThreads;
  if (wr > 65536 * 16) wr = 65536 * 16;
  pkv::launch_kernel(upload_write_kernel, dim3(static_cast<unsigned>(up + wr)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(dst),
                     reinterpret_cast<const uint4*>(dev_src), n16, static_cast<int32_t>(up),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache),
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), dev_slots,
                     total, chunks_per_token, chunks_per_row, block_size,
                     static_cast<int64_t>(num_blocks) * block_size);
  return hip_status("pkv_upload_write launch");
}
