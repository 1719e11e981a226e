// Paged prefill: causal attention of a request's new (prompt) tokens over its
// block table, on the gfx950 matrix cores.
//
// "The KV cache is a systems problem" (rsw.lol), section "Prompt processing
// and incremental decoding impose different shapes of work": the prompt phase
// attends many query tokens at once and is bound by arithmetic, decode by
// bytes.  The keys and values are read through the request's block table ("Only
// 20.4% of your KV cache held actual tokens" (blog.teqners.com), section "The
// page table, relocated into attention"), after kv_cache_write stored the
// prompt's own tokens.
//
// Request i holds L_i cached tokens; its Q_i new queries are the last Q_i
// positions, so query j sits at position L_i - Q_i + j and attends to tokens
// 0..that position (Q_i = L_i is a plain prefill; Q_i < L_i continues a cached
// prefix).
//
// One wave per work item (request, block of 16/HT queries, tile of HT query
// heads of one KV head).  The wave's 16 "columns" are (query, head) pairs,
// column c = (query j0 + c / HT, head h0 + c % HT).  Per 16-token tile:
//
//   S^T[t][c] = sum_d K[t][d] Q[c][d]     v_mfma_f32_16x16x32_f16, D/32 steps
//   O[c][d]  += sum_t P[c][t] V[t][d]     v_mfma_f32_16x16x16_f16, D/16 blocks
//
// exactly as in the decode kernel for head groups (pa_decode_mfma.hip), whose
// operand layouts this reuses: K straight from memory in the A layout, V through
// LDS and ds_read_b64_tr_b16, P from the S^T output layout rounded to fp16.
// Column c masks every token past its own position.  One pass, no split: a
// wave walks tokens [0, last position of its block + 1).
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

template <int D, int B, int HT>
__global__ __launch_bounds__(kWave) void pa_prefill_kernel(PrefillParams p) {
  constexpr int DEPTH = 2;                   // tiles in flight per wave
  constexpr int TT = 16;                     // tokens per tile
  constexpr int QB = 16 / HT;                // queries per wave
  constexpr int KSTEPS = D / 32;
  constexpr int DBLK = D / 16;
  constexpr int CPR = D / 8;
  constexpr int VLD = TT * CPR / kWave;
  constexpr int ROWB = D * 2 + 32;
  constexpr int BPT = B < TT ? TT / B : 1;
  constexpr int TPB = B > TT ? B / TT : 1;
  constexpr int CHUNKS = B * D / 8;
  static_assert(KSTEPS == VLD && (B < TT ? BPT * B == TT : TPB * TT == B), "tile shape");
  static_assert(HT == 1 || HT == 2 || HT == 4 || HT == 8 || HT == 16, "head tile");
  __shared__ __align__(16) unsigned char vlds[DEPTH][TT * ROWB];

  const int lane = threadIdx.x;
  const int grp = lane >> 4;
  const int li = lane & 15;                  // column of S^T (scores) / of O (outputs)
  const unsigned k = blockIdx.y + blockIdx.z * gridDim.y;
  if (k >= static_cast<unsigned>(p.num_items)) return;
  const uint32_t item = p.items[k];
  const int seq = static_cast<int>(item >> 16);
  const int qblk = static_cast<int>(item & 0xFFFFu);
  if (seq >= p.num_seqs) return;
  const int h0 = blockIdx.x * HT;
  const int kvh = h0 / p.group;

  const int32_t* table = p.block_tables + static_cast<int64_t>(seq) * p.max_blocks_per_seq;
  const int staged_first = lane < p.max_blocks_per_seq ? table[lane] : 0;
  const int q_first = p.q_starts[seq];
  const int nq = p.q_starts[seq + 1] - q_first;
  if (q_first < 0 || nq < 0 || q_first + nq > p.total_q) return;   // guard: bad offsets
  int len = p.context_lens[seq];
  const int cap = p.max_blocks_per_seq * B;
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int j0 = qblk * QB;
  if (j0 >= nq) return;
  const int base_pos = len - nq;             // position of query 0
  // This lane's column: query cj, head ch; its last visible token is pos.
  const int cj = j0 + li / HT;
  const int ch = h0 + li % HT;
  const bool col_ok = cj < nq;
  const int pos = col_ok ? base_pos + cj : -1;

  half8 qb[KSTEPS];
  {
    const _Float16* qp =
        p.q + (static_cast<int64_t>(q_first + (col_ok ? cj : 0)) * p.num_q_heads + ch) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const half8 v = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(qp + kk * 32));
      qb[kk] = col_ok ? v : half8{};
    }
  }
  const int j_last = min(j0 + QB, nq) - 1;
  const int t_end = min(len, base_pos + j_last + 1);   // tokens this wave reads

  float4_t o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) o[db] = float4_t{0.f, 0.f, 0.f, 0.f};
  float m = -FLT_MAX;
  float lsum = 0.f;

  if (t_end > 0) {
    const int nblk = (t_end - 1) / B + 1;
    const int ntiles = (t_end + TT - 1) / TT;
    const int64_t block_stride = static_cast<int64_t>(p.num_kv_heads) * CHUNKS;
    const uint4* kbase = p.k_cache + kvh * static_cast<int64_t>(CHUNKS);
    const uint4* vbase = p.v_cache + kvh * static_cast<int64_t>(CHUNKS);
    uint4 kbuf[DEPTH][KSTEPS], vbuf[DEPTH][VLD];

    for (int c0 = 0; c0 < nblk; c0 += kWave) {
      const int staged =
          c0 == 0 ? staged_first
                  : (lane < min(kWave, nblk - c0) && c0 + lane < p.max_blocks_per_seq
                         ? table[c0 + lane]
                         : 0);
      const int tile0 = c0 * TPB / BPT;
      const int cn = min(kWave * TPB / BPT, ntiles - tile0);

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
        for (int kk = 0; kk < KSTEPS; ++kk) kr[kk] = load_shared(kt + 4 * kk);
#pragma unroll
        for (int it = 0; it < VLD; ++it) {
          const int c = it * kWave + lane;
          locate(jj, c / CPR, raw, row);
          vr[it] = load_shared(vbase + safe(raw) * block_stride + row * CPR + c % CPR);
        }
      };

      auto consume = [&](uint4 (&kr)[KSTEPS], uint4 (&vr)[VLD], int jj, unsigned char* vl) {
        const int tok0 = (tile0 + jj) * TT;
        auto token_ok = [&](int r) {
          int raw, row;
          locate(jj, r, raw, row);
          return tok0 + r < t_end && static_cast<unsigned>(raw) < static_cast<unsigned>(p.num_blocks);
        };
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
        for (int r = 0; r < 4; ++r) {
          const int t = tok0 + 4 * grp + r;
          sr[r] = token_ok(4 * grp + r) && t <= pos ? s[r] * p.scale_log2 : -INFINITY;
        }
        float mt = fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3]));
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        const bool moved = mt > m + kSlack;
        const float m_new = moved ? mt : m;
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sr[r] - m_new);
        if (__builtin_amdgcn_ballot_w64(moved)) {
          const float alpha = fast_exp2(m - m_new);
          lsum *= alpha;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ar = shfl(alpha, 4 * grp + r);
#pragma unroll
            for (int db = 0; db < DBLK; ++db) o[db][r] *= ar;
          }
        }
        lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        m = m_new;
        const half4 pa = half4{static_cast<_Float16>(pr[0]), static_cast<_Float16>(pr[1]),
                               static_cast<_Float16>(pr[2]), static_cast<_Float16>(pr[3])};
        __syncthreads();
        const unsigned char* src = vl + (4 * grp + (li >> 2)) * ROWB + 8 * (li & 3);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          typedef __attribute__((address_space(3))) short4_t lds_short4;
          const short4_t raw =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(src + 32 * db));
          o[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(half4, raw), o[db],
                                                        0, 0, 0);
        }
      };

#pragma unroll
      for (int u = 0; u < DEPTH; ++u) issue(kbuf[u], vbuf[u], u < cn ? u : cn - 1);
      int j = 0;
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
  }

  // Denominator of column li, then each lane's output rows: columns 4*grp + r.
  float l = lsum + shfl_xor(lsum, 16);
  l = l + shfl_xor(l, 32);
  float lr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lr[r] = shfl(l, 4 * grp + r);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = 4 * grp + r;
    const int qj = j0 + c / HT;
    if (qj >= nq) continue;
    const float inv = lr[r] > 0.f ? 1.f / lr[r] : 0.f;   // a query with no token: zeros
    float* dst = p.out + (static_cast<int64_t>(q_first + qj) * p.num_q_heads + h0 + c % HT) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) dst[db * 16 + li] = o[db][r] * inv;
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
  return ht > 0 ? 16 / ht : 0;
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
  hipLaunchKernelGGL(fn, grid, dim3(kWave), dyn, static_cast<hipStream_t>(stream), prm);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pa_prefill launch: %s", hipGetErrorString(e));
  return PKV_OK;
}
