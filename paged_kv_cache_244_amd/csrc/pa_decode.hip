// pa_decode entry point: argument checks, split-context geometry and
// workspace, residency limit, launch order.  The kernel choice and the launch
// planner are host code in decode_plan.cpp.
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

#include <cfloat>
#include <cstdint>
#include <mutex>
#include <utility>
#include <vector>

#include "decode_plan.h"
#include "errors.h"
#include "launch.h"
#include "pa_decode_common.h"
#include "pagedkv.h"

namespace pkv_decode {
namespace {

// Dynamic LDS that limits a launch of fn to waves_per_cu one-wave
// workgroups per compute unit (0 = no limit).  Cached per kernel and device.
struct LdsInfo {
  const void* fn = nullptr;
  int device = -1;
  int static_bytes = 0;
  int per_cu = 0;
  int per_block = 0;
};
std::mutex g_lds_mu;
std::vector<LdsInfo> g_lds_cache;

}  // namespace

hipError_t reserve_lds_bytes(const void* fn, int waves_per_cu, unsigned* dyn) {
  *dyn = 0;
  if (waves_per_cu <= 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  LdsInfo info;
  {
    std::lock_guard<std::mutex> lock(g_lds_mu);
    for (const LdsInfo& c : g_lds_cache)
      if (c.fn == fn && c.device == dev) info = c;
  }
  if (info.fn == nullptr) {
    hipFuncAttributes attr;
    e = hipFuncGetAttributes(&attr, fn);
    if (e != hipSuccess) return e;
    info.fn = fn;
    info.device = dev;
    info.static_bytes = static_cast<int>(attr.sharedSizeBytes);
    e = hipDeviceGetAttribute(&info.per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&info.per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_lds_mu);
    g_lds_cache.push_back(info);
  }
  const int w = waves_per_cu < 4 ? 4 : waves_per_cu;
  // The workgroup's LDS total is rounded down to whole KiB: allocation is
  // granular, and a total that rounds up past per_cu / w admits one wave fewer
  // (measured: 23,296 bytes for w = 7 held 6 waves per compute unit).
  int bytes = ((info.per_cu / w) & ~1023) - info.static_bytes;
  if (bytes > info.per_block - info.static_bytes) bytes = info.per_block - info.static_bytes;
  *dyn = bytes > 0 ? static_cast<unsigned>(bytes) : 0u;
  return hipSuccess;
}

}  // namespace pkv_decode

namespace {

using pkv::fail;
using namespace pkv_decode;
using pkv_plan::KernelChoice;
using pkv_plan::align256;
using pkv_plan::choose_kernel;
using pkv_plan::parts_for;
using pkv_plan::workspace_bytes_for;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxGridY = 32768;      // work-list entries per grid row (y), then z

}  // namespace

namespace {

// Shared by both layouts.  Paged: block_tables / num_blocks / max_blocks_per_seq
// describe the table and pool.  Contiguous (row_chunks > 0): no table; num_blocks
// = max_blocks_per_seq = 16-token blocks per (request, KV head) row.
int decode_impl(float* out, const void* q, int32_t q_dtype, const void* k_cache,
                const void* v_cache, int32_t num_blocks, const int32_t* block_tables,
                int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                float scale, int32_t max_context_len, int32_t partition_size,
                const uint32_t* work_items, int32_t num_work_items, int32_t waves_per_cu,
                void* workspace, size_t workspace_bytes, void* stream, int64_t row_chunks,
                const int32_t* groups = nullptr, int32_t num_groups = 0,
                const uint32_t* group_items = nullptr, int32_t num_group_items = 0,
                const int32_t* shared_lens = nullptr, int32_t fuse = 0) {
  const bool contig = row_chunks > 0;
  const bool grouped = num_group_items > 0;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq < 0 || max_context_len < 0 || partition_size < 0 || num_work_items < 0 ||
      waves_per_cu < 0)
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
  const KernelChoice kc = choose_kernel(q_dtype, num_q_heads / num_kv_heads);
  KernelFn fn = kc.mfma ? pick_mfma_kernel(head_dim, block_size, kc.gt, contig)
                        : pick_valu_kernel(head_dim, block_size, kc.gt, q_dtype == PKV_F32, contig);
  if (!fn)
    return fail(PKV_ERR_UNSUPPORTED, "pa_decode: head_dim %d / block_size %d not built", head_dim,
                block_size);
  KernelFn group_fn = nullptr;
  if (grouped) {
    if (q_dtype != PKV_F16 || num_q_heads / num_kv_heads > 8)
      return fail(PKV_ERR_UNSUPPORTED,
                  "pa_decode_grouped: groups need fp16 q and at most 8 query heads per KV head");
    if (partition_size <= 0)
      return fail(PKV_ERR_INVALID_ARG, "pa_decode_grouped: groups need partition_size > 0");
    if (!groups || num_groups <= 0 || !group_items)
      return fail(PKV_ERR_INVALID_ARG, "pa_decode_grouped: group arrays missing");
    group_fn = pick_mfma_group_kernel(head_dim, block_size);
    if (!group_fn)
      return fail(PKV_ERR_UNSUPPORTED, "pa_decode_grouped: head_dim %d / block_size %d not built",
                  head_dim, block_size);
  }
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || (!contig && !block_tables) || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode: NULL pointer");
  const bool regular = !work_items || num_work_items > 0;
  if (!regular && !grouped) return PKV_OK;

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
  if (grouped) parts += 1;   // one spare partial slot per request (pa_decode_grouped)
  if (parts > 65535)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode: more than 65535 partitions per request");

  DecodeParams prm{};
  prm.out = out;
  prm.q = q;
  prm.k_cache = static_cast<const uint4*>(k_cache);
  prm.v_cache = static_cast<const uint4*>(v_cache);
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.items = work_items;
  prm.num_items = work_items ? num_work_items : 0;
  prm.num_seqs = num_seqs;
  prm.num_blocks = num_blocks;
  prm.max_blocks_per_seq = max_blocks_per_seq;
  prm.num_q_heads = num_q_heads;
  prm.num_kv_heads = num_kv_heads;
  prm.group = num_q_heads / num_kv_heads;
  prm.num_head_tiles = num_q_heads / kc.gt;
  prm.scale_log2 = scale * kLog2e;
  prm.len_clamp = len_clamp;
  prm.part_tokens = part_tokens;
  prm.max_parts = static_cast<int32_t>(parts);
  prm.row_chunks = row_chunks;
  prm.shared = grouped ? shared_lens : nullptr;

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

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  // Group pieces and a listed rest in one launch when the shape has a fused
  // kernel (pa_decode_fused.hip); then the reduce.
  FusedFn fused = grouped && fuse && work_items
                      ? pick_fused_kernel(head_dim, block_size, kc.gt, kc.mfma)
                      : nullptr;
  if (fused) {
    DecodeParams gp = prm;
    gp.items = group_items;
    gp.num_items = num_group_items;
    gp.groups = groups;
    gp.num_groups = num_groups;
    const int64_t group_wgs = static_cast<int64_t>(num_group_items) * num_kv_heads;
    const int64_t wgs = group_wgs + static_cast<int64_t>(num_work_items) * prm.num_head_tiles;
    if (wgs > INT32_MAX)
      return fail(PKV_ERR_INVALID_ARG, "pa_decode_grouped: %lld workgroups in one launch",
                  static_cast<long long>(wgs));
    pkv::launch_kernel(fused, dim3(static_cast<unsigned>(wgs)), dim3(kWave), 0, st, gp, prm,
                       static_cast<int>(group_wgs));
    e = hipGetLastError();
    if (e != hipSuccess)
      return fail(PKV_ERR_HIP, "pa_decode_grouped launch: %s", hipGetErrorString(e));
    e = launch_reduce(prm, head_dim, st);   // grouped launches always keep more than one slot
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_decode reduce launch: %s", hipGetErrorString(e));
    return PKV_OK;
  }
  if (grouped) {
    // Prefix groups first: their partials (or, for a member whose whole
    // context is one shared partition, its output) are in place before the
    // reduce below, which is enqueued after them on the same stream.
    DecodeParams gp = prm;
    gp.items = group_items;
    gp.num_items = num_group_items;
    gp.groups = groups;
    gp.num_groups = num_groups;
    unsigned glds = 0;
    e = reserve_lds_bytes(reinterpret_cast<const void*>(group_fn), pkv_plan::kMfmaWavesPerCu, &glds);
    if (e != hipSuccess)
      return fail(PKV_ERR_HIP, "pa_decode_grouped: kernel attributes: %s", hipGetErrorString(e));
    const int ny = num_group_items < kMaxGridY ? num_group_items : kMaxGridY;
    const dim3 ggrid(static_cast<unsigned>(num_kv_heads), static_cast<unsigned>(ny),
                     static_cast<unsigned>((num_group_items + ny - 1) / ny));
    pkv::launch_kernel(group_fn, ggrid, dim3(kWave), glds, st, gp);
    e = hipGetLastError();
    if (e != hipSuccess)
      return fail(PKV_ERR_HIP, "pa_decode_grouped launch: %s", hipGetErrorString(e));
  }

  unsigned dyn_lds = 0;
  e = reserve_lds_bytes(reinterpret_cast<const void*>(fn), waves_per_cu, &dyn_lds);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_decode: kernel attributes: %s", hipGetErrorString(e));

  // One wave per workgroup: the dispatcher then places work at wave granularity.
  // Grid x = head tile (fastest), then the pieces: with a work list, (y, z)
  // enumerate its entries in order, so the dispatcher hands out the pieces in
  // the list's order (longest first balances the compute units); without one,
  // y = request and z = partition.  Workgroups are dealt round-robin to the 8
  // XCDs and, inside an XCD, to its shader engines, so neighbours in dispatch
  // order must carry similar work: the head tiles of one piece do.
  dim3 grid(static_cast<unsigned>(prm.num_head_tiles), static_cast<unsigned>(num_seqs),
            static_cast<unsigned>(parts));
  if (work_items && num_work_items > 0) {   // an empty list (every piece grouped) launches nothing
    const int ny = num_work_items < kMaxGridY ? num_work_items : kMaxGridY;
    grid.y = static_cast<unsigned>(ny);
    grid.z = static_cast<unsigned>((num_work_items + ny - 1) / ny);
  }
  if (regular) {
    pkv::launch_kernel(fn, grid, dim3(kWave), dyn_lds, st, prm);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_decode launch: %s", hipGetErrorString(e));
  }
  if (parts > 1) {
    e = launch_reduce(prm, head_dim, st);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_decode reduce launch: %s", hipGetErrorString(e));
  }
  return PKV_OK;
}

}  // namespace

namespace pkv_decode {
// The prefill kernel's tile-pair records (pa_prefill.hip); hipErrorNotSupported
// in the product library.
hipError_t wave_timeline_read_prefill(void* dst, size_t bytes, bool clear);
}  // namespace pkv_decode

extern "C" int pkv_wave_timeline_read(int32_t kernel, void* dst, size_t bytes, int32_t clear) {
  static_assert(PKV_TIMELINE_RECORDS == kTimelineWaves && PKV_TIMELINE_WORDS == kTimelineWords,
                "timeline record layout");
  if (kernel != PKV_TIMELINE_VALU && kernel != PKV_TIMELINE_MFMA && kernel != PKV_TIMELINE_PREFILL)
    return fail(PKV_ERR_INVALID_ARG, "pkv_wave_timeline_read: unknown kernel %d", kernel);
  if (!dst && bytes > 0) return fail(PKV_ERR_INVALID_ARG, "pkv_wave_timeline_read: NULL dst");
  const hipError_t e = kernel == PKV_TIMELINE_VALU   ? wave_timeline_read_valu(dst, bytes, clear != 0)
                       : kernel == PKV_TIMELINE_MFMA ? wave_timeline_read_mfma(dst, bytes, clear != 0)
                                                     : wave_timeline_read_prefill(dst, bytes, clear != 0);
  if (e == hipErrorNotSupported)
    return fail(PKV_ERR_UNSUPPORTED,
                "pkv_wave_timeline_read: this library records no timeline (build --timeline)");
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_wave_timeline_read: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" int pa_decode(float* out, const void* q, int32_t q_dtype, const void* k_cache,
                         const void* v_cache, int32_t num_blocks, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, float scale,
                         int32_t max_context_len, int32_t partition_size,
                         const uint32_t* work_items, int32_t num_work_items, int32_t waves_per_cu,
                         void* workspace, size_t workspace_bytes, void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  return decode_impl(out, q, q_dtype, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, scale, max_context_len, partition_size, work_items,
                     num_work_items, waves_per_cu, workspace, workspace_bytes, stream, 0);
}

// ---- pa_decode_noalloc: the split-context workspace in a library-owned array ----

namespace {

// Split-context partials for pa_decode_noalloc.  Each GPU the library runs on
// holds its own copy of this array until the process ends.  In host code the
// name `scratch` is only a host-side stand-in, never a device address: kernels
// get the per-device address that hipGetSymbolAddress returns.
__device__ __align__(256) unsigned char scratch[PKV_NOALLOC_WORKSPACE_BYTES];

std::mutex g_scratch_mu;
std::vector<std::pair<int, void*>> g_scratch_addr;   // (device, address of its scratch)

// Device address of the current device's scratch array, looked up once per device
// with that device current.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_decode_noalloc: hipGetDevice: %s",
                                   hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  for (const auto& c : g_scratch_addr)
    if (c.first == dev) {
      *out = c.second;
      return PKV_OK;
    }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return fail(PKV_ERR_HIP, "pa_decode_noalloc: hipGetSymbolAddress(scratch): %s",
                hipGetErrorString(e));
  g_scratch_addr.emplace_back(dev, ptr);
  *out = ptr;
  return PKV_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(float* out, const void* q, int32_t q_dtype, const void* k_cache,
                                 const void* v_cache, int32_t num_blocks,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, float scale, int32_t max_context_len,
                                 int32_t partition_size, const uint32_t* work_items,
                                 int32_t num_work_items, int32_t waves_per_cu, void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  // The workspace this launch needs, by the same arithmetic as pa_decode's.
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq < 0 || max_context_len < 0 || partition_size < 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_noalloc: bad sizes");
  int64_t clamp64 = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  if (clamp64 > max_context_len) clamp64 = max_context_len;
  const int64_t parts = partition_size == 0
                            ? 1
                            : parts_for(static_cast<int32_t>(clamp64), partition_size);
  const size_t need = workspace_bytes_for(num_seqs, num_q_heads, head_dim, parts);
  if (need > PKV_NOALLOC_WORKSPACE_BYTES)
    return fail(PKV_ERR_WORKSPACE,
                "pa_decode_noalloc: this launch needs %zu bytes of split-context workspace, more "
                "than the library's fixed %zu; use pa_decode with a caller workspace, or a larger "
                "partition_size", need, static_cast<size_t>(PKV_NOALLOC_WORKSPACE_BYTES));
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_address(&ws);
    if (rc != PKV_OK) return rc;
  }
  return decode_impl(out, q, q_dtype, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, scale, max_context_len, partition_size, work_items,
                     num_work_items, waves_per_cu, ws, need > 0 ? PKV_NOALLOC_WORKSPACE_BYTES : 0,
                     stream, 0);
}

extern "C" int pa_decode_grouped(float* out, const void* q, int32_t q_dtype, const void* k_cache,
                                 const void* v_cache, int32_t num_blocks,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, float scale, int32_t max_context_len,
                                 int32_t partition_size, const uint32_t* work_items,
                                 int32_t num_work_items, int32_t waves_per_cu,
                                 const int32_t* groups, int32_t num_groups,
                                 const uint32_t* group_items, int32_t num_group_items,
                                 const int32_t* shared_lens, int32_t fuse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  if (num_groups < 0 || num_group_items < 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_grouped: negative group sizes");
  return decode_impl(out, q, q_dtype, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, scale, max_context_len, partition_size, work_items,
                     num_work_items, waves_per_cu, workspace, workspace_bytes, stream, 0, groups,
                     num_groups, group_items, num_group_items, shared_lens, fuse);
}

extern "C" int pa_decode_contiguous(float* out, const void* q, int32_t q_dtype,
                                    const void* k_cache, const void* v_cache, int32_t row_tokens,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    float scale, int32_t max_context_len, int32_t partition_size,
                                    const uint32_t* work_items, int32_t num_work_items,
                                    int32_t waves_per_cu, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  constexpr int32_t kTile = 16;
  if (row_tokens <= 0 || row_tokens % kTile != 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_contiguous: row_tokens %d not a positive multiple of 16",
                row_tokens);
  if (max_context_len > row_tokens)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_contiguous: max_context_len %d > row_tokens %d",
                max_context_len, row_tokens);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "pa_decode_contiguous: head_dim %d not built", head_dim);
  const int32_t blocks = row_tokens / kTile;
  return decode_impl(out, q, q_dtype, k_cache, v_cache, blocks, nullptr, blocks, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, kTile, scale, max_context_len,
                     partition_size, work_items, num_work_items, waves_per_cu, workspace,
                     workspace_bytes, stream, static_cast<int64_t>(row_tokens) * head_dim / 8);
}

