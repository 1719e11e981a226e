// Paged decode attention for query-head groups on the gfx950 matrix cores.
//
// When several query heads share one KV head ("The KV cache is a systems
// problem", section "Calculate bytes per token before choosing a batch"), each
// K/V byte read feeds GT query heads, and the VALU kernel becomes bound by its
// own arithmetic (4 heads cost ~4.7x the instructions of one).  This kernel
// moves both products of a 16-token tile onto MFMA:
//
//   S^T[t][h] = sum_d K[t][d] Q[h][d]      v_mfma_f32_16x16x32_f16, D/32 steps
//   O[h][d]  += sum_t P[h][t] V[t][d]      v_mfma_f32_16x16x16_f16, D/16 blocks
//
// Rows of the 16-wide head dimension beyond GT are zero queries (unused).  The
// output layout of S^T (lane (g, i) holds tokens 4g..4g+3 of head i) is exactly
// the A-operand layout P needs, so P goes from the softmax straight into the
// second MFMA after rounding to fp16 (P is in [0, 2^kSlack], see below).  V must be consumed with
// tokens along K, i.e. transposed relative to the pool: each V tile is written
// to LDS (rows padded by 32 bytes so the reads below hit distinct banks) and
// read back with ds_read_b64_tr_b16, which hands every lane the four tokens of
// one column.  K is loaded directly in the MFMA A layout: lane (g, i) reads
// 16 bytes of token row i at column chunk 4*kk + g.
//
// Softmax: S^T is scaled into log2 units and masked (tokens past the context
// get -inf; their V rows are zeroed in LDS).  The reference max of head i is
// kept identical in its four lane groups (the tile max crosses them with two
// lane swaps, v_permlane32_swap and v_permlane16_swap, no LDS round trip).  Rescaling is lazy: the reference max moves only when a tile's max
// exceeds it by more than kSlack = 8 (log2 units), so P = 2^(s - m) stays at
// most 2^8, where fp16 still holds it to 2^-11 relative; O and the denominator
// are rescaled only in tiles where some head's reference moved (a wave-uniform
// ballot).  Each lane accumulates its share of the denominator from the same
// fp16-rounded P that feeds the P.V product, and the four shares are summed
// once at the end.
//
// Work decomposition, masking, partitions and the workspace format are those of
// the VALU kernel in pa_decode_valu.hip, so both feed the same reduce kernel.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "pa_decode_common.h"
#include "pa_decode_mfma_body.h"

namespace pkv_decode {
namespace {

template <int D, int B, int GT, bool kContig, bool kGroups>
__global__ __launch_bounds__(kWave) void pa_decode_mfma_kernel(DecodeParams p) {
  mfma_piece<D, B, GT, kContig, kGroups>(p, launch_slot());
}

template <int D, int B, bool kContig>
KernelFn pick_gt(int gt) {
  switch (gt) {
    case 4: return pa_decode_mfma_kernel<D, B, 4, kContig, false>;
    case 8: return pa_decode_mfma_kernel<D, B, 8, kContig, false>;
    case 16: return pa_decode_mfma_kernel<D, B, 16, kContig, false>;
    default: return nullptr;
  }
}

template <int D>
KernelFn pick_b(int b, int gt) {
  switch (b) {
    case 8: return pick_gt<D, 8, false>(gt);
    case 16: return pick_gt<D, 16, false>(gt);
    case 32: return pick_gt<D, 32, false>(gt);
    case 64: return pick_gt<D, 64, false>(gt);
    case 128: return pick_gt<D, 128, false>(gt);
    default: return nullptr;
  }
}

template <int D>
KernelFn pick_group_b(int b) {
  switch (b) {
    case 8: return pa_decode_mfma_kernel<D, 8, 16, false, true>;
    case 16: return pa_decode_mfma_kernel<D, 16, 16, false, true>;
    case 32: return pa_decode_mfma_kernel<D, 32, 16, false, true>;
    case 64: return pa_decode_mfma_kernel<D, 64, 16, false, true>;
    case 128: return pa_decode_mfma_kernel<D, 128, 16, false, true>;
    default: return nullptr;
  }
}

}  // namespace

KernelFn pick_mfma_group_kernel(int head_dim, int block_size) {
  if (head_dim == 64) return pick_group_b<64>(block_size);
  if (head_dim == 128) return pick_group_b<128>(block_size);
  return nullptr;
}

KernelFn pick_mfma_kernel(int head_dim, int block_size, int gt, bool contiguous) {
  if (contiguous) {
    if (block_size != 16) return nullptr;
    if (head_dim == 64) return pick_gt<64, 16, true>(gt);
    if (head_dim == 128) return pick_gt<128, 16, true>(gt);
    return nullptr;
  }
  if (head_dim == 64) return pick_b<64>(block_size, gt);
  if (head_dim == 128) return pick_b<128>(block_size, gt);
  return nullptr;
}

hipError_t wave_timeline_read_mfma(void* dst, size_t bytes, bool clear) {
  return wave_timeline_copy(dst, bytes, clear);
}

}  // namespace pkv_decode
