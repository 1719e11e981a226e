// Paged prefill: causal attention of a request's new (prompt) tokens over its
// block table, on the gfx950 matrix cores.
//
// "The KV cache is a systems problem" (rsw.lol), section "Memory savings change
// the scheduling question", which contrasts the prompt phase with incremental
// decoding: the prompt phase attends many query tokens at once and is bound by
// arithmetic, decode by bytes.  The keys and values are read through the request's block table ("Only
// 20.4% of your KV cache held actual tokens" (blog.teqners.com), section "The
// page table, relocated into attention"), after kv_cache_write stored the
// prompt's own tokens.
//
// Request i holds L_i cached tokens; its Q_i new queries are the last Q_i
// positions, so query j sits at position L_i - Q_i + j and attends to tokens
// 0..that position (Q_i = L_i is a plain prefill; Q_i < L_i continues a cached
// prefix).
//
// One workgroup of 8 waves per work item (request, block of 8 * 2 * 16/HT
// queries, tile of HT query heads of one KV head).  The waves load each
// 64-token K/V tile once, together, into LDS (double-buffered, one barrier per
// tile), so the L2 traffic per flop is an eighth of one wave working alone.
// Measured on MI355X: 8 waves beat 4 and 16, and 64-token tiles beat 32 (half
// the barriers; every wave of the workgroup reaches each barrier).
// Each wave holds two sets of 16 "columns", (query, head) pairs: column c of
// set cs = (query wj0 + cs * 16/HT + c / HT, head h0 + c % HT).  Every K or V
// fragment a wave reads from LDS feeds one MFMA per set, which halves the LDS
// bytes per flop.  Per 16 tokens and set:
//
//   S^T[t][c] = sum_d K[t][d] Q[c][d]     v_mfma_f32_16x16x32_f16, D/32 steps
//
// and per 32 tokens and set
//
//   O[c][d]  += sum_t P[c][t] V[t][d]     v_mfma_f32_16x16x32_f16, D/16 blocks
//
// with the operand layouts of the decode kernel for head groups
// (pa_decode_mfma.hip): K read from LDS in the A layout, V through
// ds_read_b64_tr_b16 (two 4-token reads per operand), P from the S^T output
// layout rounded to fp16.  The softmax denominators come from the matrix cores
// too: the same P times a block of ones, so numerator and denominator sum the
// same rounded weights and no lane adds scores on the vector ALUs.  Column c
// masks every token past its own position; tiles that every column of a wave
// sees whole skip the masking, and a wave skips 16-token steps that lie wholly
// past its queries.  One pass, no split: the group walks tokens [0, last
// position of its block + 1).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cstdint>
#include <vector>

#include "errors.h"
#include "launch.h"
#include "pa_decode_common.h"
#include "pagedkv.h"

namespace pkv_decode {
namespace {

using pkv::fail;

struct PrefillParams {
  float* out;                   // [total_q][Hq][D]
  const _Float16* q;            // [total_q][Hq][D]
  const uint4* k_cache;         // [NB][Hkv][B][D] fp16 as 16-byte chunks
  const uint4* v_cache;
  const int32_t* block_tables;  // [S][max_blocks_per_seq]
  const int32_t* context_lens;  // [S]
  const int32_t* q_starts;      // [S + 1]
  const uint32_t* items;        // [num_items] (request << 16 | query block)
  int32_t num_items;
  int32_t total_q;
  int32_t num_seqs;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  float scale_log2;
};

constexpr float kSlack = 8.f;

// Unlike decode, every query block of a request reads the same prefix: K/V
// loads here are ordinary (cached in L2), not streaming.
__device__ __forceinline__ uint4 load_shared(const uint4* ptr) { return *ptr; }

#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 8
#endif
#ifndef PKV_PREFILL_TILE
#define PKV_PREFILL_TILE 64
#endif
#ifndef PKV_PREFILL_SETS
#define PKV_PREFILL_SETS 2
#endif
constexpr int kPrefillWaves = PKV_PREFILL_WAVES;   // waves per workgroup, sharing K/V tiles
constexpr int kPrefillSets = PKV_PREFILL_SETS;     // 16-column sets per wave, sharing LDS reads

template <int D, int B, int HT>
__global__ __launch_bounds__(kWave * kPrefillWaves) void pa_prefill_kernel(PrefillParams p) {
  constexpr int NW = kPrefillWaves;
  constexpr int NS = kPrefillSets;
  constexpr int NT = kWave * NW;             // threads
  constexpr int KT = PKV_PREFILL_TILE;       // tokens per tile (KT/16 MFMA steps)
  constexpr int SUB = KT / 16;
  constexpr int QB = 16 / HT;                // queries per set
  constexpr int QW = NS * QB;                // queries per wave
  constexpr int KSTEPS = D / 32;
  constexpr int DBLK = D / 16;
  constexpr int CPR = D / 8;                 // 16-byte chunks per token row
  // LDS bytes per K row.  Padding measured at D = 128 (SQ_LDS_BANK_CONFLICT):
  // 32 B leaves no bank conflicts, 16 B left 0.7 conflict cycles per LDS
  // instruction.  D = 64 keeps 16 B (not measured).
  constexpr int KROWB = D * 2 + (D == 128 ? 32 : 16);
  constexpr int VROWB = D * 2 + 32;          // LDS bytes per V row (transposed reads)
  constexpr int LPT = (KT * CPR + NT - 1) / NT;   // chunks of K (and V) a thread moves per tile
  constexpr int CHUNKS = B * D / 8;          // 16-byte chunks per (block, KV head)
  constexpr int TPC = kWave * B / KT;        // tiles covered by 64 staged block ids
  static_assert(LPT * NT == KT * CPR || (LPT == 1 && NT % (KT * CPR) == 0), "tile shape");
  static_assert(TPC >= 1 && TPC * KT == kWave * B, "chunk shape");
  static_assert(HT == 1 || HT == 2 || HT == 4 || HT == 8 || HT == 16, "head tile");
  static_assert(SUB % 2 == 0, "P.V takes 32 tokens per MFMA: tiles of a multiple of 32 tokens");
  __shared__ __align__(16) unsigned char klds[2][KT * KROWB];
  __shared__ __align__(16) unsigned char vlds[2][KT * VROWB];
  __shared__ __align__(4) unsigned char rowok[2][KT];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int grp = lane >> 4;
  const int li = lane & 15;                  // column of S^T (scores) / of O (outputs)
  const unsigned k = blockIdx.y + blockIdx.z * gridDim.y;
  if (k >= static_cast<unsigned>(p.num_items)) return;
  const uint32_t item = p.items[k];
  const int seq = static_cast<int>(item >> 16);
  const int sblk = static_cast<int>(item & 0xFFFFu);
  if (seq >= p.num_seqs) return;
  const int h0 = blockIdx.x * HT;
  const int kvh = h0 / p.group;

  const int32_t* table = p.block_tables + static_cast<int64_t>(seq) * p.max_blocks_per_seq;
  const int q_first = p.q_starts[seq];
  const int nq = p.q_starts[seq + 1] - q_first;
  if (q_first < 0 || nq < 0 || q_first + nq > p.total_q) return;   // guard: bad offsets
  int len = p.context_lens[seq];
  const int cap = p.max_blocks_per_seq * B;
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int j0 = sblk * NW * QW;
  if (j0 >= nq) return;
  const int base_pos = len - nq;             // position of query 0
  // This wave's queries; per set, this lane's column (query cj, head ch, last visible token pos).
  const int wj0 = j0 + wave * QW;
  const int wave_pos_max = wj0 < nq ? base_pos + min(wj0 + QW, nq) - 1 : -1;
  const int wave_pos_min = base_pos + wj0;   // every column of the wave sees tokens up to here
  const int ch = h0 + li % HT;
  int pos[NS];
  half8 qb[NS][KSTEPS];
#pragma unroll
  for (int cs = 0; cs < NS; ++cs) {
    const int cj = wj0 + cs * QB + li / HT;
    const bool col_ok = cj < nq;
    pos[cs] = col_ok ? base_pos + cj : -1;
    const _Float16* qp =
        p.q + (static_cast<int64_t>(q_first + (col_ok ? cj : 0)) * p.num_q_heads + ch) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + kk * 32);
      const unsigned mask = col_ok ? 0xFFFFFFFFu : 0u;     // component-wise: no aggregate select
      qb[cs][kk] = __builtin_bit_cast(half8, make_uint4(v.x & mask, v.y & mask, v.z & mask, v.w & mask));
    }
  }
  const int t_end = min(len, base_pos + min(j0 + NW * QW, nq));   // tokens the group reads

  // o: numerators; den: denominators, the same P times a block of ones (every
  // lane's row r of den[cs] holds the sum for column 4*grp + r of set cs).
  float4_t o[NS][DBLK], den[NS];
  float m[NS];
#pragma unroll
  for (int cs = 0; cs < NS; ++cs) {
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[cs][db] = float4_t{0.f, 0.f, 0.f, 0.f};
    den[cs] = float4_t{0.f, 0.f, 0.f, 0.f};
    m[cs] = -FLT_MAX;
  }
  const half8 ones = half8{1, 1, 1, 1, 1, 1, 1, 1};

  if (t_end > 0) {
    const int ntiles = (t_end + KT - 1) / KT;
    const int64_t block_stride = static_cast<int64_t>(p.num_kv_heads) * CHUNKS;
    const uint4* kbase = p.k_cache + kvh * static_cast<int64_t>(CHUNKS);
    const uint4* vbase = p.v_cache + kvh * static_cast<int64_t>(CHUNKS);
    struct TileRegs {
      uint4 k[LPT], v[LPT];
      bool ok[LPT];
    };
    TileRegs ra, rb;                         // two tiles in flight, in separate registers
    int staged = 0;                          // block ids of chunk `staged_chunk`, one per lane
    int staged_chunk = -1;

    // Global -> registers for tile jt: thread tid moves chunks tid, tid + NT, ...
    auto issue = [&](TileRegs& rg, int jt) __attribute__((always_inline)) {
      const int chunk = jt / TPC;
      if (chunk != staged_chunk) {           // wave-uniform: every wave stages the same ids
        const int b = chunk * kWave + lane;
        staged = b < p.max_blocks_per_seq ? table[b] : 0;
        staged_chunk = chunk;
      }
#pragma unroll
      for (int it = 0; it < LPT; ++it) {
        const int c = (it * NT + tid) % (KT * CPR);   // threads beyond the tile repeat a chunk
        const int r = c / CPR;
        const int t = jt * KT + r;
        const int raw = __builtin_bit_cast(int, shfl(__builtin_bit_cast(float, staged),
                                                     (t - chunk * kWave * B) / B));
        const bool ok = t < t_end && static_cast<unsigned>(raw) < static_cast<unsigned>(p.num_blocks);
        const int64_t off = (ok ? raw : 0) * block_stride + (t % B) * CPR + c % CPR;
        rg.k[it] = load_shared(kbase + off);
        rg.v[it] = load_shared(vbase + off);
        rg.ok[it] = ok;
      }
    };
    // Registers -> LDS buffer; invalid rows become zeros and are flagged.
    auto store = [&](const TileRegs& rg, int u) __attribute__((always_inline)) {
#pragma unroll
      for (int it = 0; it < LPT; ++it) {
        const int c = it * NT + tid;
        if (c >= KT * CPR) break;            // (only when the group has more threads than chunks)
        const int r = c / CPR;
        const unsigned mask = rg.ok[it] ? 0xFFFFFFFFu : 0u;   // component-wise: no aggregate select
        const uint4 kv = rg.k[it], vv = rg.v[it];
        *reinterpret_cast<uint4*>(&klds[u][r * KROWB + (c % CPR) * 16]) =
            make_uint4(kv.x & mask, kv.y & mask, kv.z & mask, kv.w & mask);
        *reinterpret_cast<uint4*>(&vlds[u][r * VROWB + (c % CPR) * 16]) =
            make_uint4(vv.x & mask, vv.y & mask, vv.z & mask, vv.w & mask);
        if (c % CPR == 0) rowok[u][r] = rg.ok[it] ? 1 : 0;
      }
    };
    // One wave's column sets against the KT-token tile in buffer u: every 16-token
    // score step first (each K fragment feeding every set), then per set one max
    // exchange and one softmax update for the tile, then P.V (each V fragment
    // feeding every set).
    auto compute = [&](int u, int jt) __attribute__((always_inline)) {
      const int tok0 = jt * KT;
      if (tok0 > wave_pos_max) return;       // every column of this wave is past here
      float4_t s[NS][SUB];
#pragma unroll
      for (int sub = 0; sub < SUB; ++sub) {
#pragma unroll
        for (int cs = 0; cs < NS; ++cs) s[cs][sub] = float4_t{0.f, 0.f, 0.f, 0.f};
        if (sub > 0 && tok0 + sub * 16 > wave_pos_max) continue;   // step wholly masked
        const unsigned char* krow = &klds[u][(sub * 16 + li) * KROWB + grp * 16];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const half8 kv = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(krow + kk * 64));
#pragma unroll
          for (int cs = 0; cs < NS; ++cs)
            s[cs][sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qb[cs][kk], s[cs][sub], 0, 0, 0);
        }
      }
      // Masking is needed only where some column of this wave sees part of the tile
      // (the diagonal) or some row is not a valid token (the last tile): elsewhere
      // every score enters as it is.
      const bool masked = tok0 + KT - 1 > wave_pos_min || tok0 + KT > t_end;
      if (masked) {
        unsigned ok4[SUB];                   // rows 4*grp .. 4*grp+3 of each step: validity flags
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub)
          ok4[sub] = *reinterpret_cast<const unsigned*>(&rowok[u][sub * 16 + 4 * grp]);
#pragma unroll
        for (int cs = 0; cs < NS; ++cs)
#pragma unroll
          for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = tok0 + sub * 16 + 4 * grp + r;
              const bool vis = ((ok4[sub] >> (8 * r)) & 0xFFu) != 0 && t <= pos[cs];
              s[cs][sub][r] = vis ? s[cs][sub][r] : -INFINITY;
            }
      }
      half4 pa[NS][SUB];
#pragma unroll
      for (int cs = 0; cs < NS; ++cs) {
        // Maximum of the raw scores (the scale is positive), then in log2 units.
        float mt = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub)
          mt = fmaxf(mt, fmaxf(fmaxf(s[cs][sub][0], s[cs][sub][1]), fmaxf(s[cs][sub][2], s[cs][sub][3])));
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        mt *= p.scale_log2;
        const bool moved = mt > m[cs] + kSlack;
        const float m_new = moved ? mt : m[cs];
        float pr[SUB][4];
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
          for (int r = 0; r < 4; ++r) pr[sub][r] = fast_exp2(fmaf(s[cs][sub][r], p.scale_log2, -m_new));
        if (__builtin_amdgcn_ballot_w64(moved)) {
          const float alpha = fast_exp2(m[cs] - m_new);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ar = shfl(alpha, 4 * grp + r);
            den[cs][r] *= ar;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) o[cs][db][r] *= ar;
          }
        }
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub)
          pa[cs][sub] = half4{static_cast<_Float16>(pr[sub][0]), static_cast<_Float16>(pr[sub][1]),
                              static_cast<_Float16>(pr[sub][2]), static_cast<_Float16>(pr[sub][3])};
        m[cs] = m_new;
      }
      // P.V over 32 tokens per MFMA (the double-rate 16x16x32 form): slots 0-3 of a
      // lane's operand are tokens 4*grp..4*grp+3 of one 16-token step, slots 4-7
      // the same rows of the next step, in A (probabilities) and B (transposed V)
      // alike, so the sum over k pairs each probability with its own V row.
      typedef __attribute__((address_space(3))) short4_t lds_short4;
#pragma unroll
      for (int sp = 0; sp < SUB; sp += 2) {
        const unsigned char* src0 =
            &vlds[u][(sp * 16 + 4 * grp + (li >> 2)) * VROWB + 8 * (li & 3)];
        const unsigned char* src1 = src0 + 16 * VROWB;
        half8 pa8[NS];
#pragma unroll
        for (int cs = 0; cs < NS; ++cs)
          pa8[cs] = half8{pa[cs][sp][0], pa[cs][sp][1], pa[cs][sp][2], pa[cs][sp][3],
                          pa[cs][sp + 1][0], pa[cs][sp + 1][1], pa[cs][sp + 1][2], pa[cs][sp + 1][3]};
#pragma unroll
        for (int cs = 0; cs < NS; ++cs)
          den[cs] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa8[cs], ones, den[cs], 0, 0, 0);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const half4 v0 = __builtin_bit_cast(
              half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(src0 + 32 * db)));
          const half4 v1 = __builtin_bit_cast(
              half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(src1 + 32 * db)));
          const half8 vf = half8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int cs = 0; cs < NS; ++cs)
            o[cs][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa8[cs], vf, o[cs][db], 0, 0, 0);
        }
      }
    };

    // Tile jt is in register set ra (even jt) or rb (odd jt) and LDS buffer jt % 2.
    auto step = [&](TileRegs& rg, int u, int jt) __attribute__((always_inline)) {
      store(rg, u);
      if (jt + 2 < ntiles) issue(rg, jt + 2);
      __syncthreads();                       // tile jt visible; the other buffer free again
      compute(u, jt);
    };
    issue(ra, 0);
    if (ntiles > 1) issue(rb, 1);
    int jt = 0;
    for (; jt + 1 < ntiles; jt += 2) {
      step(ra, 0, jt);
      step(rb, 1, jt + 1);
    }
    if (jt < ntiles) step(ra, 0, jt);
  }

  // Per set: each lane's output rows, columns 4*grp + r, over their denominators.
#pragma unroll
  for (int cs = 0; cs < NS; ++cs) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 4 * grp + r;
      const int qj = wj0 + cs * QB + c / HT;
      if (qj >= nq) continue;
      const float inv = den[cs][r] > 0.f ? 1.f / den[cs][r] : 0.f;   // a query with no token: zeros
      float* dst = p.out + (static_cast<int64_t>(q_first + qj) * p.num_q_heads + h0 + c % HT) * D;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) dst[db * 16 + li] = o[cs][db][r] * inv;
    }
  }
}

using PrefillFn = void (*)(PrefillParams);

template <int D, int B>
PrefillFn pick_ht(int ht) {
  switch (ht) {
    case 1: return pa_prefill_kernel<D, B, 1>;
    case 2: return pa_prefill_kernel<D, B, 2>;
    case 4: return pa_prefill_kernel<D, B, 4>;
    case 8: return pa_prefill_kernel<D, B, 8>;
    case 16: return pa_prefill_kernel<D, B, 16>;
    default: return nullptr;
  }
}

template <int D>
PrefillFn pick_b(int b, int ht) {
  switch (b) {
    case 8: return pick_ht<D, 8>(ht);
    case 16: return pick_ht<D, 16>(ht);
    case 32: return pick_ht<D, 32>(ht);
    case 64: return pick_ht<D, 64>(ht);
    case 128: return pick_ht<D, 128>(ht);
    default: return nullptr;
  }
}

// Query heads per wave for a group of G query heads per KV head: all of them
// up to 16 (G must divide 16 or be a multiple of 16).
int head_tile_for(int group) {
  if (group >= 16) return group % 16 == 0 ? 16 : 0;
  return 16 % group == 0 ? group : 0;
}

constexpr int kMaxGridY = 32768;
constexpr int kPrefillWavesPerCu = 0;

}  // namespace
}  // namespace pkv_decode

using pkv::fail;
using namespace pkv_decode;

extern "C" int32_t pa_prefill_queries_per_item(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  const int ht = head_tile_for(num_q_heads / num_kv_heads);
  return ht > 0 ? kPrefillWaves * kPrefillSets * 16 / ht : 0;
}

extern "C" int pa_prefill_plan(const int32_t* q_lens, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               uint32_t* items, int32_t items_capacity, int32_t* num_items_out) {
  if (!num_items_out) return fail(PKV_ERR_INVALID_ARG, "pa_prefill_plan: NULL num_items_out");
  *num_items_out = 0;
  if (num_seqs < 0 || num_seqs > 65535 || items_capacity < 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_prefill_plan: bad sizes");
  const int32_t qb = pa_prefill_queries_per_item(num_q_heads, num_kv_heads);
  if (qb == 0)
    return fail(PKV_ERR_UNSUPPORTED, "pa_prefill_plan: %d query heads over %d KV heads not built",
                num_q_heads, num_kv_heads);
  if (num_seqs > 0 && (!q_lens || !context_lens))
    return fail(PKV_ERR_INVALID_ARG, "pa_prefill_plan: NULL lengths");
  // Cost of a block = tokens its wave reads = position of its last query + 1.
  std::vector<uint64_t> keys;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t nq = q_lens[s] > 0 ? q_lens[s] : 0;
    const int64_t len = context_lens[s] > 0 ? context_lens[s] : 0;
    const int64_t nblocks = (nq + qb - 1) / qb;
    if (nblocks > 65536)
      return fail(PKV_ERR_INVALID_ARG, "pa_prefill_plan: request %d has too many query blocks", s);
    for (int64_t b = 0; b < nblocks; ++b) {
      const int64_t last = std::min<int64_t>((b + 1) * qb, nq) - 1;
      int64_t cost = len - nq + last + 1;
      cost = cost < 0 ? 0 : (cost > len ? len : cost);
      keys.push_back((static_cast<uint64_t>(UINT32_MAX - static_cast<uint32_t>(cost)) << 32) |
                     (static_cast<uint64_t>(s) << 16) | static_cast<uint64_t>(b));
    }
  }
  *num_items_out = static_cast<int32_t>(keys.size());
  if (static_cast<int64_t>(keys.size()) > items_capacity)
    return fail(PKV_ERR_INVALID_ARG, "pa_prefill_plan: %zu items do not fit in %d", keys.size(),
                items_capacity);
  if (!keys.empty() && !items) return fail(PKV_ERR_INVALID_ARG, "pa_prefill_plan: NULL items");
  std::sort(keys.begin(), keys.end());
  for (size_t i = 0; i < keys.size(); ++i) items[i] = static_cast<uint32_t>(keys[i] & 0xFFFFFFFFu);
  return PKV_OK;
}

extern "C" int pa_prefill(float* out, const void* q, const int32_t* q_starts, int32_t total_q,
                          const void* k_cache, const void* v_cache, int32_t num_blocks,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                          const uint32_t* work_items, int32_t num_work_items, void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  if (num_seqs < 0 || num_seqs > 65535 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || num_work_items < 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_prefill: bad sizes");
  if (num_q_heads % num_kv_heads != 0 || num_q_heads > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "pa_prefill: %d query heads over %d KV heads", num_q_heads,
                num_kv_heads);
  const int ht = head_tile_for(num_q_heads / num_kv_heads);
  PrefillFn fn = nullptr;
  if (ht > 0) {
    if (head_dim == 64) fn = pick_b<64>(block_size, ht);
    if (head_dim == 128) fn = pick_b<128>(block_size, ht);
  }
  if (!fn)
    return fail(PKV_ERR_UNSUPPORTED, "pa_prefill: head_dim %d / block_size %d / group %d not built",
                head_dim, block_size, num_q_heads / num_kv_heads);
  if (num_seqs == 0 || total_q == 0 || num_work_items == 0) return PKV_OK;
  if (!out || !q || !q_starts || !k_cache || !v_cache || !block_tables || !context_lens ||
      !work_items)
    return fail(PKV_ERR_INVALID_ARG, "pa_prefill: NULL pointer");

  PrefillParams prm{};
  prm.out = out;
  prm.q = static_cast<const _Float16*>(q);
  prm.k_cache = static_cast<const uint4*>(k_cache);
  prm.v_cache = static_cast<const uint4*>(v_cache);
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.q_starts = q_starts;
  prm.items = work_items;
  prm.num_items = num_work_items;
  prm.total_q = total_q;
  prm.num_seqs = num_seqs;
  prm.num_blocks = num_blocks;
  prm.max_blocks_per_seq = max_blocks_per_seq;
  prm.num_q_heads = num_q_heads;
  prm.num_kv_heads = num_kv_heads;
  prm.group = num_q_heads / num_kv_heads;
  prm.scale_log2 = scale * 1.4426950408889634f;

  unsigned dyn = 0;
  hipError_t e = reserve_lds_bytes(reinterpret_cast<const void*>(fn), kPrefillWavesPerCu, &dyn);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_prefill: kernel attributes: %s", hipGetErrorString(e));
  const int ny = num_work_items < kMaxGridY ? num_work_items : kMaxGridY;
  const dim3 grid(static_cast<unsigned>(num_q_heads / ht), static_cast<unsigned>(ny),
                  static_cast<unsigned>((num_work_items + ny - 1) / ny));
  pkv::launch_kernel(fn, grid, dim3(kWave * kPrefillWaves), dyn, static_cast<hipStream_t>(stream),
                     prm);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_prefill launch: %s", hipGetErrorString(e));
  return PKV_OK;
}
