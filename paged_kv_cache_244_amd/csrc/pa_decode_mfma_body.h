// Body of the MFMA decode kernel for query-head groups (and, in group mode,
// for prefix groups of requests), as a device function over an explicit
// launch position so that more than one launch shape can run it
// (pa_decode_mfma.hip, pa_decode_fused.hip).  The design notes are in
// pa_decode_mfma.hip.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "pa_decode_common.h"

namespace pkv_decode {

constexpr float kSlack = 8.f;

// kGroups: the launch runs prefix groups (GT is 16): the tile's rows are the
// query heads of several requests that read the same physical blocks over the
// piece's tokens, so each K/V tile is read once for all of them.  The block
// table and length of the group's first member describe the piece.
template <int D, int B, int GT, bool kContig, bool kGroups>
__device__ __forceinline__ void mfma_piece(const DecodeParams& p, PieceSlot slot) {
#ifndef PKV_MFMA_DEPTH
#define PKV_MFMA_DEPTH 2
#endif
  constexpr int DEPTH = PKV_MFMA_DEPTH;      // tiles in flight per wave
  constexpr int TT = 16;                     // tokens per tile
  constexpr int KSTEPS = D / 32;             // score MFMAs per tile
  constexpr int DBLK = D / 16;               // P.V MFMAs per tile
  constexpr int CPR = D / 8;                 // 16-byte chunks per token row
  constexpr int VLD = TT * CPR / kWave;      // wave-wide loads per V tile
  constexpr int ROWB = D * 2 + 32;           // LDS bytes per V row (padded)
  constexpr int BPT = B < TT ? TT / B : 1;   // blocks per tile
  constexpr int TPB = B > TT ? B / TT : 1;   // tiles per block
  constexpr int CHUNKS = B * D / 8;          // 16-byte chunks per (block, KV head)
  static_assert(KSTEPS == VLD && (B < TT ? BPT * B == TT : TPB * TT == B), "tile shape");
  static_assert(GT == 4 || GT == 8 || GT == 16, "head group");
  __shared__ __align__(16) unsigned char vlds[DEPTH][TT * ROWB];

  WaveTimeline tl;                           // empty unless built with PKV_WAVE_TIMELINE
  const int lane = threadIdx.x;
  const int grp = lane >> 4;                 // lane group: tokens 4*grp..4*grp+3 of a tile
  const int li = lane & 15;                  // head index (scores) / column (outputs)
  int seq, part;                             // seq: the request, or the group (kGroups)
  if (!scheduled_piece_at(p, slot.y, slot.z, slot.gdy, seq, part,
                          kGroups ? p.num_groups : p.num_seqs))
    return;
  tl.entry();
  // Tile row r: query head h0 + r of request seq; with groups, query head
  // h0 + r % G of member r / G.  Rows at or past `rows` are unused.
  int h0, kvh, rows, rep;
  const int32_t* members = nullptr;
  if constexpr (kGroups) {
    kvh = spread_column(slot.x, p.num_kv_heads);
    h0 = kvh * p.group;
    members = p.groups + static_cast<int64_t>(seq) * kGroupStride + 1;
    const int cap = GT / p.group;            // members that fit in the tile
    const int n = members[-1];
    rows = (n < 1 ? 1 : (n > cap ? cap : n)) * p.group;
  } else {
    h0 = spread_column(slot.x, p.num_head_tiles) * GT;
    kvh = h0 / p.group;
    rows = GT;
  }
  // Request and query head of tile row r (r < rows); member ids out of range read as 0.
  auto row_seq = [&](int r) {
    if constexpr (kGroups) {
      const int m = members[r / p.group];
      return static_cast<unsigned>(m) < static_cast<unsigned>(p.num_seqs) ? m : 0;
    } else {
      return seq;
    }
  };
  auto row_head = [&](int r) { return kGroups ? h0 + r % p.group : h0 + r; };
  rep = row_seq(0);

  // Independent loads first: table ids, queries, length.
  const int32_t* table =
      kContig ? nullptr : p.block_tables + static_cast<int64_t>(rep) * p.max_blocks_per_seq;
  const int blk_begin = part * (p.part_tokens / B);
  const int staged_first = block_id<kContig>(table, blk_begin + lane, p.max_blocks_per_seq);
  half8 qb[KSTEPS];                          // Q^T as the B operand: head li, dims kk*32 + 8*grp
  {
    const int r = li < rows ? li : 0;
    const _Float16* qp = static_cast<const _Float16*>(p.q) +
                         (static_cast<int64_t>(row_seq(r)) * p.num_q_heads + row_head(r)) * D +
                         8 * grp;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const half8 v = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(qp + kk * 32));
      qb[kk] = li < rows ? v : half8{};
    }
  }
  const int len = clamped_len(p, rep);
  const int shared = shared_len(p, rep);
  tl.inputs();
  const int t_begin = part * p.part_tokens;
  if (t_begin >= len) {
    if (!kGroups && part == 0) {              // empty context: defined as zeros
      float* const out_rows = p.out + (static_cast<int64_t>(seq) * p.num_q_heads + h0) * D;
      for (int x = lane; x < GT * D / 4; x += kWave)
        reinterpret_cast<float4*>(out_rows)[x] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  // A shared prefix that ends inside this partition splits it: a group piece
  // takes the tokens before that point, a request's own piece the rest (from
  // a block boundary, so whole tiles are skipped and, with 8-token blocks, the
  // first tile is masked up to it), its partial kept in the spare slot.
  const bool split = shared > t_begin && shared < t_begin + p.part_tokens;
  const int t_first = !kGroups && split ? shared : t_begin;
  const int t_end = min(kGroups && split ? shared : len, t_begin + p.part_tokens);
  if (t_first >= t_end) return;               // no tokens of its own here
  const int nparts = (len + p.part_tokens - 1) / p.part_tokens;
  const int skip_tiles = (t_first - t_begin) / TT;
  const int nblk = (t_end - 1) / B - blk_begin + 1;
  const int ntiles = (t_end - t_begin + TT - 1) / TT;
  const TileAddressing<kContig, CHUNKS> at(p, seq, kvh);
  const int64_t block_stride = at.block_stride;
  const uint4* kbase = p.k_cache + at.head_base;
  const uint4* vbase = p.v_cache + at.head_base;

  float4_t o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) o[db] = float4_t{0.f, 0.f, 0.f, 0.f};
  float m = -FLT_MAX;     // running max of head li (log2 units), equal in all lane groups
  float lsum = 0.f;       // this lane's share of head li's denominator

  uint4 kbuf[DEPTH][KSTEPS], vbuf[DEPTH][VLD];

  for (int c0 = 0; c0 < nblk; c0 += kWave) {
    const int staged =
        c0 == 0 ? staged_first
                : (lane < min(kWave, nblk - c0)
                       ? block_id<kContig>(table, blk_begin + c0 + lane, p.max_blocks_per_seq)
                       : 0);
    const int tile0 = c0 * TPB / BPT;                         // first tile of this chunk
    const int cn = min(kWave * TPB / BPT, ntiles - tile0);    // tiles in this chunk
    const int j0 = skip_tiles > tile0 ? skip_tiles - tile0 : 0;   // first tile to compute
    if (j0 >= cn) continue;

    // Physical block (raw table entry) and row inside it of token row r of tile jj.
    auto locate = [&](int jj, int r, int& raw, int& row) {
      if constexpr (BPT == 1) {
        raw = __builtin_amdgcn_readlane(staged, jj / TPB);
        row = (jj % TPB) * TT + r;
      } else {
        const int first = __builtin_amdgcn_readlane(staged, jj * BPT);
        const int second = __builtin_amdgcn_readlane(staged, jj * BPT + 1);
        raw = r < B ? first : second;
        row = r % B;
      }
    };
    auto safe = [&](int raw) {
      return static_cast<unsigned>(raw) < static_cast<unsigned>(p.num_blocks) ? raw : 0;
    };

    auto issue = [&](uint4 (&kr)[KSTEPS], uint4 (&vr)[VLD], int jj) {
      int raw, row;
      locate(jj, li, raw, row);
      const uint4* kt = kbase + safe(raw) * block_stride + row * CPR + grp;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) kr[kk] = load_stream(kt + 4 * kk);
#pragma unroll
      for (int it = 0; it < VLD; ++it) {
        const int c = it * kWave + lane;
        locate(jj, c / CPR, raw, row);
        vr[it] = load_stream(vbase + safe(raw) * block_stride + row * CPR + c % CPR);
      }
    };

    auto consume = [&](uint4 (&kr)[KSTEPS], uint4 (&vr)[VLD], int jj, unsigned char* vl) {
      tl.first_tile();
      const int tok0 = t_begin + (tile0 + jj) * TT;
      auto token_ok = [&](int r) {
        int raw, row;
        locate(jj, r, raw, row);
        return tok0 + r >= t_first && tok0 + r < t_end &&
               static_cast<unsigned>(raw) < static_cast<unsigned>(p.num_blocks);
      };
      // V tile into LDS first (its latency hides behind the score MFMAs).
#pragma unroll
      for (int it = 0; it < VLD; ++it) {
        const int c = it * kWave + lane;
        const int r = c / CPR;
        const uint4 v = token_ok(r) ? vr[it] : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(vl + r * ROWB + (c % CPR) * 16) = v;
      }
      float4_t s = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, kr[kk]), qb[kk], s, 0,
                                                  0, 0);
      float sr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sr[r] = token_ok(4 * grp + r) ? s[r] * p.scale_log2 : -INFINITY;
      float mt = column_max(fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3])));
      // Lazy rescaling: the reference max of a head moves only when a score
      // exceeds it by more than kSlack (log2 units), so P stays below 2^kSlack
      // (exact enough in fp16) and the accumulators are rescaled rarely.
      const bool moved = mt > m + kSlack;
      const float m_new = moved ? mt : m;
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sr[r] - m_new);
      if (__builtin_amdgcn_ballot_w64(moved)) {    // some head moved: rescale (wave-uniform)
        const float alpha = fast_exp2(m - m_new);
        lsum *= alpha;
        // O rows are heads 4*grp + r; head h's factor lives in lane h.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = shfl(alpha, 4 * grp + r);
#pragma unroll
          for (int db = 0; db < DBLK; ++db) o[db][r] *= ar;
        }
      }
      m = m_new;
      const half4 pa = half4{static_cast<_Float16>(pr[0]), static_cast<_Float16>(pr[1]),
                             static_cast<_Float16>(pr[2]), static_cast<_Float16>(pr[3])};
      // The denominator sums the same fp16-rounded weights the P.V product uses,
      // so numerator and denominator carry one rounding.
      lsum += (static_cast<float>(pa[0]) + static_cast<float>(pa[1])) +
              (static_cast<float>(pa[2]) + static_cast<float>(pa[3]));
      __syncthreads();                        // V tile visible in LDS
      const unsigned char* src = vl + (4 * grp + (li >> 2)) * ROWB + 8 * (li & 3);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        typedef __attribute__((address_space(3))) short4_t lds_short4;
        const short4_t raw =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(src + 32 * db));
        o[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(half4, raw), o[db], 0,
                                                      0, 0);
      }
    };

#pragma unroll
    for (int u = 0; u < DEPTH; ++u) issue(kbuf[u], vbuf[u], j0 + u < cn ? j0 + u : cn - 1);
    int j = j0;
    for (; j + 2 * DEPTH - 1 < cn; j += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        consume(kbuf[u], vbuf[u], j + u, vlds[u]);
        issue(kbuf[u], vbuf[u], j + u + DEPTH);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      if (j + u < cn) consume(kbuf[u], vbuf[u], j + u, vlds[u]);
      if (j + u + DEPTH < cn) issue(kbuf[u], vbuf[u], j + u + DEPTH);
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
      if (j + u + DEPTH < cn) consume(kbuf[u], vbuf[u], j + u + DEPTH, vlds[u]);
  }

  tl.finish(slot, ntiles - skip_tiles, seq, part, t_end - t_first);
  // Denominator of head li: the four lane groups' shares.
  float l = lsum + shfl_xor(lsum, 16);
  l = l + shfl_xor(l, 32);
  float lr[4], mr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {               // this lane's output rows: heads 4*grp + r
    lr[r] = shfl(l, 4 * grp + r);
    mr[r] = shfl(m, 4 * grp + r);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * grp + r;
    if (h >= rows) continue;
    // A member's own partition count decides whether this piece is its whole
    // context (write the output) or one of several partials.
    const int rs = row_seq(h);
    int np = nparts, own_slot = !kGroups && split ? nparts : part;
    if constexpr (kGroups) {
      const int rl = clamped_len(p, rs);
      np = partials_of((rl + p.part_tokens - 1) / p.part_tokens, shared_len(p, rs), rl);
    } else {
      np = partials_of(nparts, shared, len);
    }
    const int64_t orow = static_cast<int64_t>(rs) * p.num_q_heads + row_head(h);
    if (np == 1) {
      const float inv = 1.f / lr[r];
#pragma unroll
      for (int db = 0; db < DBLK; ++db) p.out[orow * D + db * 16 + li] = o[db][r] * inv;
    } else {
      const int64_t slot = orow * p.max_parts + own_slot;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) p.ws_o[slot * D + db * 16 + li] = o[db][r];
      if (li == 0) {
        p.ws_ml[2 * slot] = mr[r];
        p.ws_ml[2 * slot + 1] = lr[r];
      }
    }
  }
}

}  // namespace pkv_decode
