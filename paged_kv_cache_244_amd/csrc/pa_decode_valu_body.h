// Body of the VALU decode kernel (one query head, or a small head group, per
// wave), as a device function over an explicit launch position so that more
// than one launch shape can run it (pa_decode_valu.hip, pa_decode_fused.hip).
// Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "pa_decode_common.h"

namespace pkv_decode {

// ---- the partition kernel -------------------------------------------------------

template <int GT, bool kQF32>
struct QueryRegs;

template <int GT>
struct QueryRegs<GT, true> {        // fp32 queries: fp32 FMA with the fp16 keys widened in place
  float v[GT][8];
  __device__ __forceinline__ void load(const void* q, int64_t base, int64_t head_stride) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float4* ptr = reinterpret_cast<const float4*>(static_cast<const float*>(q) + base +
                                                          g * head_stride);
      float4 a = ptr[0], b = ptr[1];
      v[g][0] = a.x; v[g][1] = a.y; v[g][2] = a.z; v[g][3] = a.w;
      v[g][4] = b.x; v[g][5] = b.y; v[g][6] = b.z; v[g][7] = b.w;
    }
  }
  __device__ __forceinline__ float dot(int g, uint4 k) const {
    half8 kh = __builtin_bit_cast(half8, k);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(v[g][i], static_cast<float>(kh[i]), acc);
    return acc;
  }
};

template <int GT>
struct QueryRegs<GT, false> {       // fp16 queries: v_dot2_f32_f16 (products exact in fp32)
  half2_t v[GT][4];
  __device__ __forceinline__ void load(const void* q, int64_t base, int64_t head_stride) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const _Float16*>(q) + base +
                                                  g * head_stride);
      v[g][0] = __builtin_bit_cast(half2_t, raw.x);
      v[g][1] = __builtin_bit_cast(half2_t, raw.y);
      v[g][2] = __builtin_bit_cast(half2_t, raw.z);
      v[g][3] = __builtin_bit_cast(half2_t, raw.w);
    }
  }
  __device__ __forceinline__ float dot(int g, uint4 k) const {
    float acc = __builtin_amdgcn_fdot2(v[g][0], __builtin_bit_cast(half2_t, k.x), 0.f, false);
    acc = __builtin_amdgcn_fdot2(v[g][1], __builtin_bit_cast(half2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2(v[g][2], __builtin_bit_cast(half2_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2(v[g][3], __builtin_bit_cast(half2_t, k.w), acc, false);
    return acc;
  }
};

// One (request, head tile, partition) piece on one wave; `slot` is the
// workgroup's (virtual) position in its launch.
template <int D, int B, int GT, bool kQF32, bool kContig>
__device__ __forceinline__ void valu_piece(const DecodeParams& p, PieceSlot slot) {
  constexpr int LPT = D / 8;               // lanes per token row
  constexpr int TPL = kWave / LPT;         // token rows per wave-wide load
  // Pipeline unit: a tile of TT tokens of one (block, KV head), at most 4 KiB, so
  // register use does not grow with the block size.  A block is TPB tiles.
  constexpr int TT = B < 2048 / D ? B : 2048 / D;
  constexpr int TPB = B / TT;
  constexpr int NLD = TT * D / 8 / kWave;  // wave-wide loads per tile
  constexpr int CHUNKS = B * D / 8;        // 16-byte chunks per (block, KV head)
  static_assert(NLD >= 1 && NLD * TPL == TT && TPB * TT == B, "tile shape");

  WaveTimeline tl;                         // empty unless built with PKV_WAVE_TIMELINE
  const int lane = threadIdx.x & (kWave - 1);
  const int tile = spread_column(slot.x, p.num_head_tiles);
  int seq, part;
  if (!scheduled_piece_at(p, slot.y, slot.z, slot.gdy, seq, part, p.num_seqs)) return;
  tl.entry();
  const int h0 = tile * GT;
  const int kvh = h0 / p.group;
  const int row = lane / LPT;
  const int dchunk = lane % LPT;

  // The first 64 block ids of this partition, the query and the length do not
  // depend on one another: issue all three loads before waiting on any.
  const int32_t* table =
      kContig ? nullptr : p.block_tables + static_cast<int64_t>(seq) * p.max_blocks_per_seq;
  const int blk_begin = part * (p.part_tokens / B);
  const int staged_first = block_id<kContig>(table, blk_begin + lane, p.max_blocks_per_seq);
  QueryRegs<GT, kQF32> qr;
  qr.load(p.q, (static_cast<int64_t>(seq) * p.num_q_heads + h0) * D + dchunk * 8, D);
  const int len = clamped_len(p, seq);
  const int shared = shared_len(p, seq);
  tl.inputs();
  const int t_begin = part * p.part_tokens;
  if (t_begin >= len) {
    if (part == 0 && row == 0) {             // empty context: defined as zeros
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float4* o = reinterpret_cast<float4*>(
            p.out + (static_cast<int64_t>(seq) * p.num_q_heads + h0 + g) * D + dchunk * 8);
        o[0] = make_float4(0.f, 0.f, 0.f, 0.f);
        o[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }
  const int t_end = min(len, t_begin + p.part_tokens);
  const int nparts = (len + p.part_tokens - 1) / p.part_tokens;
  // When the request's shared prefix ends inside this partition, a group
  // piece has its tokens before that point: start there (block-aligned, so a
  // whole number of tiles in) and keep the partial in the spare slot.
  const bool own_rest = shared > t_begin && shared < t_begin + p.part_tokens;
  const int skip_tiles = own_rest ? (shared - t_begin) / TT : 0;
  if (own_rest && shared >= t_end) return;   // no tokens of its own here
  const int slot_part = own_rest ? nparts : part;
  const int np_eff = partials_of(nparts, shared, len);

  float m[GT], l[GT], o[GT][8];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = -FLT_MAX;
    l[g] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[g][k] = 0.f;
  }

  const int nblk = (t_end - 1) / B - blk_begin + 1;
  const int ntiles = (t_end - t_begin + TT - 1) / TT;
  const TileAddressing<kContig, CHUNKS> at(p, seq, kvh);
  const int64_t block_stride = at.block_stride;
  const uint4* kbase = p.k_cache + at.head_base + lane;
  const uint4* vbase = p.v_cache + at.head_base + lane;

  // DEPTH tiles in flight per wave: while one tile of K and V is consumed, the
  // loads of the next DEPTH-1 are outstanding.  Three for one head per wave; two
  // when a wave serves a head group (register pressure).
  constexpr int DEPTH = GT == 1 ? 3 : 2;
  uint4 kbuf[DEPTH][NLD], vbuf[DEPTH][NLD];

  // Blocks are taken 64 at a time (one id per lane); tiles are numbered from the
  // start of the partition.
  for (int c0 = 0; c0 < nblk; c0 += kWave) {
    const int staged =
        c0 == 0 ? staged_first
                : (lane < min(kWave, nblk - c0)
                       ? block_id<kContig>(table, blk_begin + c0 + lane, p.max_blocks_per_seq)
                       : 0);
    const int tile0 = c0 * TPB;                               // first tile of this chunk
    const int cn = min(kWave * TPB, ntiles - tile0);          // tiles in this chunk
    const int j0 = skip_tiles > tile0 ? skip_tiles - tile0 : 0;   // first tile to compute
    if (j0 >= cn) continue;

    auto issue = [&](uint4 (&kr)[NLD], uint4 (&vr)[NLD], int jj) {
      int ph = __builtin_amdgcn_readlane(staged, jj / TPB);
      ph = static_cast<unsigned>(ph) < static_cast<unsigned>(p.num_blocks) ? ph : 0;
      const int64_t off = ph * block_stride + (jj % TPB) * (TT * D / 8);
      const uint4* kt = kbase + off;
      const uint4* vt = vbase + off;
#pragma unroll
      for (int it = 0; it < NLD; ++it) kr[it] = load_stream(kt + it * kWave);
#pragma unroll
      for (int it = 0; it < NLD; ++it) vr[it] = load_stream(vt + it * kWave);
    };

    auto consume = [&](uint4 (&kr)[NLD], uint4 (&vr)[NLD], int jj) {
      tl.first_tile();
      const int ph = __builtin_amdgcn_readlane(staged, jj / TPB);
      const bool blk_ok = static_cast<unsigned>(ph) < static_cast<unsigned>(p.num_blocks);
      const int tok0 = t_begin + (tile0 + jj) * TT + row;
      float s[GT][NLD];
#pragma unroll
      for (int it = 0; it < NLD; ++it) {
        const bool valid = blk_ok && (tok0 + it * TPL < t_end);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const float acc = row_sum<LPT>(qr.dot(g, kr[it])) * p.scale_log2;
          s[g][it] = valid ? acc : -INFINITY;
        }
        if (!valid) vr[it] = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float mb = s[g][0];
#pragma unroll
        for (int it = 1; it < NLD; ++it) mb = fmaxf(mb, s[g][it]);
        const float m_new = fmaxf(m[g], mb);
        const float alpha = fast_exp2(m[g] - m_new);
        l[g] *= alpha;
#pragma unroll
        for (int k = 0; k < 8; ++k) o[g][k] *= alpha;
#pragma unroll
        for (int it = 0; it < NLD; ++it) {
          const float pr = fast_exp2(s[g][it] - m_new);
          l[g] += pr;
          half8 vh = __builtin_bit_cast(half8, vr[it]);
#pragma unroll
          for (int k = 0; k < 8; ++k) o[g][k] = fmaf(pr, static_cast<float>(vh[k]), o[g][k]);
        }
        m[g] = m_new;
      }
    };

    // Prologue issues are unconditional (a short chunk re-reads its last tile,
    // an L2 hit) so every path into the loop has the same DEPTH tiles in flight
    // and the compiler waits for exactly the tile it consumes.
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) issue(kbuf[u], vbuf[u], j0 + u < cn ? j0 + u : cn - 1);
    int j = j0;
    for (; j + 2 * DEPTH - 1 < cn; j += DEPTH) {   // steady state: unconditional issues
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        consume(kbuf[u], vbuf[u], j + u);
        issue(kbuf[u], vbuf[u], j + u + DEPTH);
        __builtin_amdgcn_sched_barrier(0);   // keep the refill ahead of the next tile's math
      }
    }
    // At most 2*DEPTH-1 tiles remain; buffer u holds tile j+u when that exists.
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      if (j + u < cn) consume(kbuf[u], vbuf[u], j + u);
      if (j + u + DEPTH < cn) issue(kbuf[u], vbuf[u], j + u + DEPTH);
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
      if (j + u + DEPTH < cn) consume(kbuf[u], vbuf[u], j + u + DEPTH);
  }

  // Merge the TPL token rows: lanes with equal dchunk differ by multiples of LPT.
#pragma unroll
  for (int mask = LPT; mask < kWave; mask <<= 1) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float m2 = shfl_xor(m[g], mask);
      const float l2 = shfl_xor(l[g], mask);
      const float mm = fmaxf(m[g], m2);
      const float a = fast_exp2(m[g] - mm);
      const float b = fast_exp2(m2 - mm);
      l[g] = l[g] * a + l2 * b;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[g][k] = o[g][k] * a + shfl_xor(o[g][k], mask) * b;
      m[g] = mm;
    }
  }

  tl.finish(slot, ntiles - skip_tiles, seq, part, t_end - t_begin - skip_tiles * TT);
  if (row != 0) return;
  if (np_eff == 1) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float inv = 1.f / l[g];
      float4* dst = reinterpret_cast<float4*>(
          p.out + (static_cast<int64_t>(seq) * p.num_q_heads + h0 + g) * D + dchunk * 8);
      dst[0] = make_float4(o[g][0] * inv, o[g][1] * inv, o[g][2] * inv, o[g][3] * inv);
      dst[1] = make_float4(o[g][4] * inv, o[g][5] * inv, o[g][6] * inv, o[g][7] * inv);
    }
  } else {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const int64_t slot =
          (static_cast<int64_t>(seq) * p.num_q_heads + h0 + g) * p.max_parts + slot_part;
      float4* dst = reinterpret_cast<float4*>(p.ws_o + slot * D + dchunk * 8);
      dst[0] = make_float4(o[g][0], o[g][1], o[g][2], o[g][3]);
      dst[1] = make_float4(o[g][4], o[g][5], o[g][6], o[g][7]);
      if (dchunk == 0) {
        p.ws_ml[2 * slot] = m[g];
        p.ws_ml[2 * slot + 1] = l[g];
      }
    }
  }
}

}  // namespace pkv_decode
