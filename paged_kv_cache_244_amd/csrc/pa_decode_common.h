// Definitions shared by the two pa_decode kernel families (VALU and MFMA):
// launch parameters and cross-lane helpers.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "pagedkv.h"

namespace pkv_decode {

constexpr int kWave = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

struct DecodeParams {
  float* out;                 // [S][Hq][D]
  float* ws_o;                // [S][Hq][max_parts][D]  unnormalised partial outputs
  float* ws_ml;               // [S][Hq][max_parts][2]  (running max in log2 units, sum)
  const void* q;              // [S][Hq][D], fp32 or fp16
  const uint4* k_cache;       // [NB][Hkv][B][D] fp16 viewed as 16-byte chunks
  const uint4* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const uint32_t* items;      // optional [num_items] (request << 16 | partition), NULL = grid
  int32_t num_seqs;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;              // num_q_heads / num_kv_heads
  int32_t num_head_tiles;     // num_q_heads / GT
  float scale_log2;           // scale * log2(e)
  int32_t len_clamp;          // min(max_context_len, max_blocks_per_seq * B)
  int32_t part_tokens;        // tokens per partition, multiple of B
  int32_t max_parts;
  int32_t num_items;
  int64_t row_chunks;         // contiguous layout only: 16-byte chunks per (request, KV head) row
  const int32_t* groups;      // group launches: [num_groups][kGroupStride] (count, requests...)
  int32_t num_groups;
  const int32_t* shared;      // group launches: [S] shared length ending inside a partition, or 0; may be NULL
};

// A prefix group (pagedkv.h, pa_decode_grouped): requests whose first tokens
// are stored in the same physical blocks.  Row i of the descriptor array: the
// member count, then the members' request indices.
constexpr int kGroupStride = PKV_GROUP_STRIDE;

// Where the tiles of one (request, KV head) live.  Paged: block id b (from the
// table) of KV head g starts at chunk (b * Hkv + g) * CHUNKS.  Contiguous
// ([S][Hkv][Lmax][D], the layout without a block table): logical block b of
// (request s, KV head g) starts at chunk (s * Hkv + g) * row_chunks + b * CHUNKS,
// so the "block id" is the logical block number itself.
template <bool kContig, int CHUNKS>
struct TileAddressing {
  int64_t head_base;      // chunk offset of block 0 of this (request, KV head)
  int64_t block_stride;   // chunks between consecutive block ids
  __device__ TileAddressing(const DecodeParams& p, int seq, int kvh) {
    if constexpr (kContig) {
      head_base = (static_cast<int64_t>(seq) * p.num_kv_heads + kvh) * p.row_chunks;
      block_stride = CHUNKS;
    } else {
      head_base = static_cast<int64_t>(kvh) * CHUNKS;
      block_stride = static_cast<int64_t>(p.num_kv_heads) * CHUNKS;
    }
  }
};

// Block id of logical block `blk` of the request: its table entry (paged), or
// blk itself (contiguous); ids past the table read as 0 (never used unguarded).
template <bool kContig>
__device__ __forceinline__ int block_id(const int32_t* table, int blk, int max_blocks) {
  if constexpr (kContig) return blk;
  return blk < max_blocks ? table[blk] : 0;
}

// K/V tiles are read exactly once: non-temporal loads keep them from displacing
// useful lines in L2 and the Infinity Cache (measured ~10% faster on MI355X).
__device__ __forceinline__ uint4 load_stream(const uint4* ptr) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Sum over the LPT lanes of one token row; every lane of the row gets the same
// bits (each step adds two equal-order partial sums).
template <int LPT>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: pairs
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: quads
  v += dpp<0x141>(v);   // row_half_mirror: 8 lanes
  if constexpr (LPT == 16) v += dpp<0x140>(v);   // row_mirror: 16 lanes
  return v;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  const int lane = __lane_id();
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float shfl(float v, int src_lane) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Which head tile (or KV head) workgroup column x serves.  The dispatcher deals
// workgroups to the 8 XCDs in turn, and the grid's x extent n is the fastest
// index, so when n is a multiple of 8 column 8q + k always lands on XCD k.  With
// the identity, XCD k would read only the heads of residue k mod 8, whose tiles
// sit at a fixed offset in every block; on MI355X the XCDs that drew the odd
// residues then ran ~20% slower per tile (OPT-13B, 40 heads).  Rotating the
// residue by q gives every XCD heads of every residue.  A bijection of [0, n).
__device__ __forceinline__ int spread_column(int x, int n) {
  return n % 8 == 0 ? (x & ~7) | (((x & 7) + (x >> 3)) & 7) : x;
}

// Maximum over the four lanes of a column (lanes l, l ^ 16, l ^ 32, l ^ 48).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second, v_permlane16_swap the odd rows of the first with
// the even rows of the second; with both operands holding v, every lane finds
// its partner's value in one of the two results.  The second operand is an
// identity DPP move of v rather than v itself: given two identical operands the
// compiler takes the two results to be equal and drops one.
__device__ __forceinline__ float swap_max(float v, bool halves) {
  const int b = __builtin_bit_cast(int, v);
  const int c = __builtin_amdgcn_mov_dpp(b, 0xE4, 0xF, 0xF, false);   // quad_perm [0,1,2,3]
  const auto x = halves ? __builtin_amdgcn_permlane32_swap(b, c, false, false)
                        : __builtin_amdgcn_permlane16_swap(b, c, false, false);
  return fmaxf(v, fmaxf(__builtin_bit_cast(float, static_cast<int>(x[0])),
                        __builtin_bit_cast(float, static_cast<int>(x[1]))));
}

__device__ __forceinline__ float column_max(float v) {
  return swap_max(swap_max(v, true), false);
}

// The (request, partition) piece handled by this workgroup.  With a work list,
// grid (y, z) enumerates its entries in order (y fastest); without one, grid y
// is the request and z the partition.  Returns false for entries to skip.
// by, bz, gdy: the workgroup's (virtual) grid y and z and the grid's y extent.
__device__ __forceinline__ bool scheduled_piece_at(const DecodeParams& p, unsigned by, unsigned bz,
                                                   unsigned gdy, int& seq, int& part, int limit) {
  if (p.items) {
    const unsigned k = by + bz * gdy;
    if (k >= static_cast<unsigned>(p.num_items)) return false;
    const uint32_t it = p.items[k];
    seq = static_cast<int>(it >> 16);
    part = static_cast<int>(it & 0xFFFFu);
  } else {
    seq = static_cast<int>(by);
    part = static_cast<int>(bz);
  }
  return seq < limit && part < p.max_parts;
}

// A workgroup's position in a launch of one kernel family: grid x (head tile,
// or KV head for groups) and the work-list coordinates.
struct PieceSlot {
  int x;
  unsigned y, z, gdy;
};

__device__ __forceinline__ PieceSlot launch_slot() {
  return PieceSlot{static_cast<int>(blockIdx.x), blockIdx.y, blockIdx.z, gridDim.y};
}

__device__ __forceinline__ int clamped_len(const DecodeParams& p, int seq) {
  const int len = p.context_lens[seq];
  return len < 0 ? 0 : (len > p.len_clamp ? p.len_clamp : len);
}

// Shared length of request seq when it ends inside a partition (group
// launches), else 0.
__device__ __forceinline__ int shared_len(const DecodeParams& p, int seq) {
  return p.shared ? p.shared[seq] : 0;
}

// Partials request seq (of length len) combines: one per partition, plus a
// spare (slot nparts) for its own tokens of the partition its shared length
// ends in, when it has tokens past that length.  One partial means the piece
// writes the output itself.
__device__ __forceinline__ int partials_of(int nparts, int shared, int len) {
  return nparts + (shared > 0 && len > shared ? 1 : 0);
}

// Per-wave timeline of the decode kernels, for measurement only.  It is compiled
// in with -DPKV_WAVE_TIMELINE (the instrumented library libpagedkv_timeline.so,
// `python -m paged_kv_cache_244_amd.build --timeline`); in the product library
// every member below is empty and the kernels are unchanged.  Each wave that
// streams a piece writes one record of six 64-bit words into the array of its
// translation unit, at its position in the launch (work-list entry * grid x +
// column); pkv_wave_timeline_read copies the array to the host:
//   0, 1  real-time counter (100 MHz) at the wave's start and at its end
//   2     shader-clock cycles from the start to the work-list entry (bits 0-31)
//         and to the table row, query and length (bits 32-63)
//   3     cycles to the first tile consumed (bits 0-31) and to the end (32-63)
//   4     XCC id (bits 0-31) and tiles of the piece (bits 32-63)
//   5     request or group (bits 0-19), partition (20-39), tokens (40-63)
// The two start-up marks wait for every load in flight, so the instrumented
// start-up overlaps its loads at most as much as the product's.
constexpr int kTimelineWaves = 16384;
constexpr int kTimelineWords = 6;
#ifdef PKV_WAVE_TIMELINE
static __device__ uint64_t g_wave_timeline[kTimelineWaves * kTimelineWords];

struct WaveTimeline {
  uint64_t rt0, c0, c1 = 0, c2 = 0, c3 = 0;
  __device__ __forceinline__ WaveTimeline()
      : rt0(__builtin_amdgcn_s_memrealtime()), c0(__builtin_amdgcn_s_memtime()) {}
  __device__ __forceinline__ void entry() {
    __builtin_amdgcn_s_waitcnt(0);
    c1 = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void inputs() {
    __builtin_amdgcn_s_waitcnt(0);
    c2 = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void first_tile() {
    if (c3 == 0) c3 = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void finish(PieceSlot slot, int ntiles, int seq, int part,
                                         int tokens) {
    const uint64_t c4 = __builtin_amdgcn_s_memtime();
    const uint64_t rt1 = __builtin_amdgcn_s_memrealtime();
    const unsigned xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // XCC_ID, 32 bits
    const unsigned idx = (slot.y + slot.z * slot.gdy) * gridDim.x + static_cast<unsigned>(slot.x);
    if ((threadIdx.x & (kWave - 1)) != 0 || idx >= static_cast<unsigned>(kTimelineWaves)) return;
    auto since = [&](uint64_t c) { return c ? (c - c0) & 0xFFFFFFFFull : 0ull; };
    uint64_t* r = g_wave_timeline + static_cast<uint64_t>(idx) * kTimelineWords;
    r[0] = rt0;
    r[1] = rt1;
    r[2] = since(c1) | (since(c2) << 32);
    r[3] = since(c3) | (since(c4) << 32);
    r[4] = static_cast<uint64_t>(xcc) | (static_cast<uint64_t>(ntiles) << 32);
    r[5] = (static_cast<uint64_t>(seq) & 0xFFFFF) | ((static_cast<uint64_t>(part) & 0xFFFFF) << 20) |
           (static_cast<uint64_t>(tokens) << 40);
  }
};

// This translation unit's records to the host (at most the array's size), then,
// with `clear`, zeroed.  Synchronous.
static inline hipError_t wave_timeline_copy(void* dst, size_t bytes, bool clear) {
  const size_t cap = sizeof(g_wave_timeline);
  hipError_t e = hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_wave_timeline), bytes < cap ? bytes : cap, 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess || !clear) return e;
  void* addr = nullptr;
  e = hipGetSymbolAddress(&addr, HIP_SYMBOL(g_wave_timeline));
  if (e != hipSuccess) return e;
  return hipMemset(addr, 0, cap);
}
#else
struct WaveTimeline {
  __device__ __forceinline__ void entry() {}
  __device__ __forceinline__ void inputs() {}
  __device__ __forceinline__ void first_tile() {}
  __device__ __forceinline__ void finish(PieceSlot, int, int, int, int) {}
};

static inline hipError_t wave_timeline_copy(void*, size_t, bool) { return hipErrorNotSupported; }
#endif

// Host side of the timeline: copy the records of the VALU (pa_decode_valu.hip)
// or MFMA (pa_decode_mfma.hip) translation unit to dst and, with `clear`, zero
// them.  hipErrorNotSupported in the product library.
hipError_t wave_timeline_read_valu(void* dst, size_t bytes, bool clear);
hipError_t wave_timeline_read_mfma(void* dst, size_t bytes, bool clear);

// MFMA head-group kernel, defined in pa_decode_mfma.hip: 16-token tiles, scores
// on v_mfma_f32_16x16x32_f16 and P.V on v_mfma_f32_16x16x16_f16, for head
// groups of GT in {4, 8, 16} query heads and fp16 queries.
using KernelFn = void (*)(DecodeParams);
KernelFn pick_mfma_kernel(int head_dim, int block_size, int gt, bool contiguous);

// The same kernel over prefix groups (pa_decode_grouped): a work item is
// (group, partition), grid x the KV head, and the 16 rows of the tile are
// (member i / G, query head i % G) pairs, G = num_q_heads / num_kv_heads.
KernelFn pick_mfma_group_kernel(int head_dim, int block_size);

// Group pieces and remaining pieces in one launch (pa_decode_fused.hip):
// grid x = group_wgs + remaining workgroups; arguments (group launch
// parameters, remaining-piece parameters, group_wgs).  gt and mfma name the
// remaining pieces' kernel as the shape alone would use it.
using FusedFn = void (*)(DecodeParams, DecodeParams, int);
FusedFn pick_fused_kernel(int head_dim, int block_size, int gt, bool mfma);

// VALU kernel (pa_decode_valu.hip): one wave per (request, head tile,
// partition), GT in {1, 2, 4} query heads per wave, fp32 or fp16 queries.
// `contiguous` selects the layout without a block table (block size 16 only).
KernelFn pick_valu_kernel(int head_dim, int block_size, int gt, bool qf32, bool contiguous);

// Cross-partition combine (pa_decode_reduce.hip), launched after a split pass.
hipError_t launch_reduce(const DecodeParams& prm, int head_dim, hipStream_t stream);

}  // namespace pkv_decode
