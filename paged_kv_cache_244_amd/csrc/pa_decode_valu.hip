// VALU decode kernel: one query head (or a small group with fp32 queries) per
// wave, scores and P.V on the vector ALUs.  See pa_decode.hip for the entry
// point and the launch geometry.
//
// What is computed: "800 kilobytes per token" (shashforge.dev), section "The old
// answer, imported honestly", and "Only 20.4% of your KV cache held actual
// tokens" (blog.teqners.com), section "The page table, relocated into
// attention": attention whose kernel walks a per-request table of fixed-size
// physical blocks instead of one contiguous tensor.  The decode step is a
// matrix-vector product per request and is bound by memory (teqners, section
// "Why the KV cache is the thing that limits your batch"), so this kernel is an
// HBM-streaming kernel: no MFMA, fp32 VALU arithmetic on fp16 data.
//
// Work decomposition (one wave64 per work item):
//   item = (request, head tile, partition).  A head tile is GT query heads that
//   share one KV head ("The KV cache is a systems problem", section "Calculate
//   bytes per token before choosing a batch"), so every K/V tile is read once
//   per tile.  A partition is part_tokens consecutive logical tokens
//   (block-aligned); long contexts split into several partitions that run in
//   parallel and are merged by pa_decode_reduce with a log-sum-exp combine.
//   Each work item is its own one-wave workgroup; requests are dispatched in
//   the caller's work order (longest first balances the CUs best).
//
// Lane layout: one (block, KV head) region of B tokens x D halves is contiguous
// in the pool and is read as tiles of TT <= 2048/D tokens (at most 4 KiB).  A
// tile is read as 16-byte chunks, chunk c = it*64 + lane, so one wave-wide load
// covers TPL = 64 / (D/8) consecutive tokens and lane holds dims
// [(lane % LPT)*8, +8) of token it*TPL + lane / LPT.  Loads are fully coalesced
// 1 KiB wave transactions, issued DEPTH tiles ahead of use (software pipeline).
// A score is the sum over the LPT lanes of a token row, reduced with DPP row
// permutations (no LDS).
//
// Softmax: each token row (the LPT lanes that share lane / LPT) keeps its own
// running max, sum and output for the tokens it sees; rows are merged once at
// the end of the partition with cross-lane shuffles.  Scores are kept in the
// log2 domain (q . k * scale * log2 e) so exp2 (v_exp_f32) is used directly.
// Masked tokens (past the context length) get score -inf and their value
// vectors are replaced by zeros with a select, so stale or NaN slots never leak.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "pa_decode_common.h"
#include "pa_decode_valu_body.h"

namespace pkv_decode {
namespace {

template <int D, int B, int GT, bool kQF32, bool kContig>
__global__ __launch_bounds__(kWave) void pa_decode_partition_kernel(DecodeParams p) {
  valu_piece<D, B, GT, kQF32, kContig>(p, launch_slot());
}

template <int D, int B, int GT, bool kContig>
KernelFn pick_q(bool qf32) {
  return qf32 ? pa_decode_partition_kernel<D, B, GT, true, kContig>
              : pa_decode_partition_kernel<D, B, GT, false, kContig>;
}

template <int D, int B, bool kContig>
KernelFn pick_gt(int gt, bool qf32) {
  switch (gt) {
    case 1: return pick_q<D, B, 1, kContig>(qf32);
    case 2: return pick_q<D, B, 2, kContig>(qf32);
    case 4: return pick_q<D, B, 4, kContig>(qf32);
    default: return nullptr;
  }
}

template <int D>
KernelFn pick_b(int b, int gt, bool qf32) {
  switch (b) {
    case 8: return pick_gt<D, 8, false>(gt, qf32);
    case 16: return pick_gt<D, 16, false>(gt, qf32);
    case 32: return pick_gt<D, 32, false>(gt, qf32);
    case 64: return pick_gt<D, 64, false>(gt, qf32);
    case 128: return pick_gt<D, 128, false>(gt, qf32);
    default: return nullptr;
  }
}

}  // namespace

KernelFn pick_valu_kernel(int head_dim, int block_size, int gt, bool qf32, bool contiguous) {
  if (contiguous) {
    if (block_size != 16) return nullptr;
    if (head_dim == 64) return pick_gt<64, 16, true>(gt, qf32);
    if (head_dim == 128) return pick_gt<128, 16, true>(gt, qf32);
    return nullptr;
  }
  if (head_dim == 64) return pick_b<64>(block_size, gt, qf32);
  if (head_dim == 128) return pick_b<128>(block_size, gt, qf32);
  return nullptr;
}

hipError_t wave_timeline_read_valu(void* dst, size_t bytes, bool clear) {
  return wave_timeline_copy(dst, bytes, clear);
}

}  // namespace pkv_decode
