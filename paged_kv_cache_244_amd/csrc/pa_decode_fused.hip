// One launch for a grouped decode (pa_decode_grouped): the prefix-group pieces
// and the remaining pieces share one grid.  The first group_wgs workgroups
// run group pieces (the MFMA body in group mode, one per (group piece, KV
// head)); the rest run the remaining pieces on the body the shape uses
// alone (VALU with GT query heads per wave, or MFMA for head groups of 4 or
// more).  The two kinds write different partial slots, so they need no
// ordering between them; the reduce launched after this kernel merges both.
// In separate launches the short group launch and the many short remaining
// pieces each leave the GPU partly idle, and a gap separates them; here the
// dispatcher fills the slots the long group waves leave free.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_decode_common.h"
#include "pa_decode_mfma_body.h"
#include "pa_decode_valu_body.h"

namespace pkv_decode {
namespace {

template <int D, int B, int GT, bool kMfma>
__global__ __launch_bounds__(kWave) void pa_decode_fused_kernel(DecodeParams pg, DecodeParams pr,
                                                                 int group_wgs) {
  const int lin = static_cast<int>(blockIdx.x);
  if (lin < group_wgs) {
    const int hk = pg.num_kv_heads;
    mfma_piece<D, B, 16, false, true>(pg, PieceSlot{lin % hk, static_cast<unsigned>(lin / hk), 0u, 1u});
  } else {
    const int r = lin - group_wgs;
    const int tiles = pr.num_head_tiles;
    const PieceSlot slot{r % tiles, static_cast<unsigned>(r / tiles), 0u, 1u};
    if constexpr (kMfma)
      mfma_piece<D, B, GT, false, false>(pr, slot);
    else
      valu_piece<D, B, GT, false, false>(pr, slot);   // groups come with fp16 queries
  }
}

template <int D, int B>
FusedFn pick_regular(int gt, bool mfma) {
  if (mfma) {
    switch (gt) {
      case 4: return pa_decode_fused_kernel<D, B, 4, true>;
      case 8: return pa_decode_fused_kernel<D, B, 8, true>;
      default: return nullptr;
    }
  }
  switch (gt) {
    case 1: return pa_decode_fused_kernel<D, B, 1, false>;
    case 2: return pa_decode_fused_kernel<D, B, 2, false>;
    case 4: return pa_decode_fused_kernel<D, B, 4, false>;
    default: return nullptr;
  }
}

template <int D>
FusedFn pick_fused_b(int b, int gt, bool mfma) {
  switch (b) {
    case 8: return pick_regular<D, 8>(gt, mfma);
    case 16: return pick_regular<D, 16>(gt, mfma);
    case 32: return pick_regular<D, 32>(gt, mfma);
    case 64: return pick_regular<D, 64>(gt, mfma);
    case 128: return pick_regular<D, 128>(gt, mfma);
    default: return nullptr;
  }
}

}  // namespace

FusedFn pick_fused_kernel(int head_dim, int block_size, int gt, bool mfma) {
  if (head_dim == 64) return pick_fused_b<64>(block_size, gt, mfma);
  if (head_dim == 128) return pick_fused_b<128>(block_size, gt, mfma);
  return nullptr;
}

}  // namespace pkv_decode
