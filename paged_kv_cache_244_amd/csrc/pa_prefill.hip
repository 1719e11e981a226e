// Paged prefill: causal attention of a request's new (prompt) tokens over its
// block table, on the gfx950 matrix cores.
//
// "The KV cache is a systems problem" (rsw.lol), section "Memory savings change
// the scheduling question", which contrasts the prompt phase with incremental
// decoding: the prompt phase attends many query tokens at once and is bound by
// arithmetic, decode by bytes.  The keys and values are read through the
// request's block table ("Only 20.4% of your KV cache held actual tokens"
// (blog.teqners.com), section "The page table, relocated into attention"),
// after kv_cache_write stored the prompt's own tokens.
//
// Request i holds L_i cached tokens; its Q_i new queries are the last Q_i
// positions, so query j sits at position L_i - Q_i + j and attends to tokens
// 0..that position (Q_i = L_i is a plain prefill; Q_i < L_i continues a cached
// prefix).
//
// One workgroup of 8 waves per work item (request, block of 8 * 2 * 16/HT
// queries, tile of HT query heads of one KV head).  Each wave holds two sets of
// 16 "columns", (query, head) pairs: column c of set cs = (query wj0 + cs *
// 16/HT + c / HT, head h0 + c % HT).  Per 16 tokens and set
//
//   S^T[t][c] = sum_d K[t][d] Q[c][d]     v_mfma_f32_16x16x32_f16, D/32 steps
//
// and per 32 tokens and set
//
//   O[c][d]  += sum_t P[c][t] V[t][d]     v_mfma_f32_16x16x32_f16, D/16 blocks
//
// with K read from LDS in the A layout, V through ds_read_b64_tr_b16 (two
// 4-token reads per operand) and P taken from the S^T output layout rounded to
// fp16.  The softmax denominators come from the matrix cores too (the same P
// times a block of ones), so numerator and denominator sum the same rounded
// weights.
//
// Keys and values move by 64-token tiles straight from memory into LDS
// (buffer loads with an LDS destination: no registers, no vector-ALU work).
// A load group is 8 rows of a tile, which lie in one cache block; its buffer
// resource spans only those rows of that block, so rows past the last token
// the workgroup reads are out of range and arrive as zeros.  Rows are
// unpadded; the 16-byte chunks of row r are stored XOR-permuted by a function
// of r so that the 16 rows one K fragment read touches, and the rows of a V
// transposed read, fall on distinct LDS banks.
//
// Waves 0-3 and 4-7 (one of each per SIMD) alternate between two phases per
// tile, one phase apart: the matrix phase (P.V of the previous tile, then the
// scores of this tile) and the softmax phase (mask, maximum, exponentials,
// rare rescale) on the vector ALUs; the probabilities are rounded to fp16 in
// the matrix phase that uses them, which is the shorter one.  While one wave of a SIMD
// keeps the matrix core busy the other runs its softmax, and every tile pair
// (two phases) ends at a workgroup barrier.  Two K and two V tile buffers.  The waves in their
// softmax phase issue the loads, each two row groups: K(m+1) by waves 4-7 at
// the start of phase 2m, V(m) by waves 0-3 at the start of phase 2m+1, both
// waited for before the barrier that ends phase 2m+1.

// Column c masks every token past its own position; tiles that every column of
// a wave sees whole skip the masking, and a wave skips tiles that lie wholly
// past its queries.  One pass, no split: the workgroup walks tokens [0, last
// position of its block + 1).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cstdint>
#include <type_traits>
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
constexpr int kPrefillWaves = 8;   // waves per workgroup, sharing K/V tiles
constexpr int kPrefillSets = 2;    // 16-column sets per wave, sharing LDS reads
constexpr int kPrefillTile = 64;   // tokens per K/V tile
constexpr int kPvAhead = 3;        // P.V steps whose V operands are read ahead

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4_t lds_short4;

// Word 3 of a buffer resource for plain byte-addressed (raw) access on gfx9-family GPUs.
constexpr int kRawBufferWord3 = 0x00020000;
// s_waitcnt operand: every outstanding vector-memory load done (vmcnt 0), the
// other counters left unconstrained.  Loads into LDS count as vector-memory loads.
constexpr int kWaitVmem = 0x0F70;

// Logical 16-byte chunk c of tile row r sits at chunk c ^ lds_swizzle<D>(r) of
// the row.  D = 128 (256-byte rows, one per 64-bank line): XOR with r mod 16
// puts the 16 rows of a K fragment read on 16 distinct chunks, and the four
// rows of a transposed V read (two chunks each) on distinct chunk pairs; of
// the permutations tried it read fastest in a transposed-read probe on gfx950.
// D = 64 (128-byte rows, two per line): XOR with 2 ((r/2) mod 4) + (r/8 mod 2)
// gives the 16 rows of a K read 16 distinct (half-line, chunk) slots and the 8
// rows of a V read distinct 32-byte slots.  Either way the swizzle depends on
// r mod 16 only.
template <int D>
__device__ __forceinline__ int lds_swizzle(int r) {
  if constexpr (D == 128) {
    return r & 15;
  } else {
    const int q = r >> 1;
    return 2 * (q & 3) + ((q >> 2) & 1);
  }
}

// Wave-wide load of n (1 or 2) x 1 KiB from src straight into LDS at dst: load
// i writes bytes [i * 1024, (i + 1) * 1024) of dst, lane l's 16 bytes at offset
// l * 16 of them, read from src + voff_i.  Offsets at or past `bytes` are out of
// range: no memory is read and zeros land in LDS.  src, bytes and dst must be
// the same in every lane of the wave; the first-lane reads keep the compiler
// from building the buffer resource in vector registers.  (A plain device
// function: the buffer-resource type has no host form.)
__device__ __forceinline__ void load_rows(const unsigned char* src, int bytes, unsigned char* dst,
                                          unsigned voff0, unsigned voff1, int n) {
  // readfirstlane yields a signed int: each half goes through unsigned before it
  // is widened, so the low half never sign-extends into the high one.
  const uint64_t a = reinterpret_cast<uint64_t>(src);
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
  const uint64_t a_s = (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(a_s), 0, __builtin_amdgcn_readfirstlane(bytes), kRawBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff0, 0, 0, 0);
  if (n > 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + 1024), 16, voff1, 0, 0, 0);
}

// Tile-pair timeline of the prefill kernel, for measurement only: compiled in
// with -DPKV_WAVE_TIMELINE (libpagedkv_timeline.so), empty otherwise.  Each
// wave of a full 64-query workgroup of head tile 0 sums, over tile pairs 8-39,
// the shader-clock cycles of seven stretches of a pair: 0 from the end of the
// previous pair to this one's start; 1 its first-half load issue; 2 its
// first-half work; 3 between the halves (no barrier there); 4 its second-half
// load issue; 5 its second-half work; 6 its wait for its loads.  The barrier ending
// the pair falls in stretch 0 of the next.  Record (pkv_wave_timeline_read,
// PKV_TIMELINE_PREFILL), at work item * 8 + wave: stretches 0-5 as 32-bit
// pairs in words 0-2, stretch 6 and the pairs summed in word 3, the work item
// and the wave in word 4, the XCC id in word 5.
#ifdef PKV_WAVE_TIMELINE
static __device__ uint64_t g_prefill_timeline[kTimelineWaves * kTimelineWords];

struct PairClock {
  uint64_t ts[7], acc[7] = {0, 0, 0, 0, 0, 0, 0}, prev = 0;
  uint32_t pairs = 0;
  __device__ __forceinline__ void mark(int i) { ts[i] = __builtin_amdgcn_s_memtime(); }
  __device__ __forceinline__ void end_pair(int mm) {
    if (mm >= 8 && mm < 40) {
      acc[0] += ts[0] - prev;
#pragma unroll
      for (int i = 1; i < 7; ++i) acc[i] += ts[i] - ts[i - 1];
      ++pairs;
    }
    prev = ts[6];
  }
  __device__ __forceinline__ void finish(unsigned item, int wave, bool full) {
    const unsigned idx = item * kPrefillWaves + static_cast<unsigned>(wave);
    if (blockIdx.x != 0 || !full || (threadIdx.x & (kWave - 1)) != 0 ||
        idx >= static_cast<unsigned>(kTimelineWaves))
      return;
    auto lo = [](uint64_t v) { return v & 0xFFFFFFFFull; };
    uint64_t* r = g_prefill_timeline + static_cast<uint64_t>(idx) * kTimelineWords;
    r[0] = lo(acc[0]) | (lo(acc[1]) << 32);
    r[1] = lo(acc[2]) | (lo(acc[3]) << 32);
    r[2] = lo(acc[4]) | (lo(acc[5]) << 32);
    r[3] = lo(acc[6]) | (static_cast<uint64_t>(pairs) << 32);
    r[4] = static_cast<uint64_t>(item) | (static_cast<uint64_t>(wave) << 32);
    r[5] = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // XCC_ID
  }
};

static hipError_t prefill_timeline_copy(void* dst, size_t bytes, bool clear) {
  const size_t cap = sizeof(g_prefill_timeline);
  hipError_t e = hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_prefill_timeline), bytes < cap ? bytes : cap,
                                     0, hipMemcpyDeviceToHost);
  if (e != hipSuccess || !clear) return e;
  void* addr = nullptr;
  e = hipGetSymbolAddress(&addr, HIP_SYMBOL(g_prefill_timeline));
  if (e != hipSuccess) return e;
  return hipMemset(addr, 0, cap);
}
#else
struct PairClock {
  __device__ __forceinline__ void mark(int) {}
  __device__ __forceinline__ void end_pair(int) {}
  __device__ __forceinline__ void finish(unsigned, int, bool) {}
};

static hipError_t prefill_timeline_copy(void*, size_t, bool) { return hipErrorNotSupported; }
#endif

template <int D, int B, int HT>
__global__ __launch_bounds__(kWave * kPrefillWaves) void pa_prefill_kernel(PrefillParams p) {
  constexpr int NW = kPrefillWaves;
  constexpr int NS = kPrefillSets;
  constexpr int KT = kPrefillTile;
  constexpr int SUB = KT / 16;               // 16-token score steps per tile
  constexpr int QB = 16 / HT;                // queries per set
  constexpr int QW = NS * QB;                // queries per wave
  constexpr int KSTEPS = D / 32;
  constexpr int DBLK = D / 16;
  constexpr int CPR = D / 8;                 // 16-byte chunks per token row
  constexpr int ROWB = 2 * D;                // bytes per token row, in memory and in LDS
  constexpr int TILEB = KT * ROWB;
  constexpr int RPW = KT / NW;               // tile rows each wave loads
  constexpr int RPI = kWave * 16 / ROWB;     // rows one wave-wide 16-byte-per-lane load covers
  constexpr int NI = RPW / RPI;              // such loads per wave, tile and tensor
  static_assert(RPW % RPI == 0 && B % RPW == 0, "a wave's rows of a tile lie in one block");
  static_assert(NI == 1 || NI == 2, "load_rows moves one or two 1 KiB pieces");
  static_assert(HT == 1 || HT == 2 || HT == 4 || HT == 8 || HT == 16, "head tile");
  static_assert(SUB % 2 == 0, "P.V takes 32 tokens per MFMA: tiles of a multiple of 32 tokens");
  __shared__ __align__(256) unsigned char kt0[TILEB], kt1[TILEB], vt0[TILEB], vt1[TILEB];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
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

  // Waves 0-3 run their matrix phases on even phases, waves 4-7 on odd ones.
  // Each group gets its own copy of the schedule, so that no value one order
  // needs is kept alive through the other's code.
  auto run = [&](auto odd_phases) __attribute__((always_inline)) {
    constexpr bool XO = decltype(odd_phases)::value;
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

    if (t_end > 0) {
      const int n = (t_end + KT - 1) / KT;     // tiles
      // Last tile this wave attends to (-1: none); wave-uniform.
      const int last = wave_pos_max >= 0 ? min(n - 1, wave_pos_max / KT) : -1;
      const half8 ones = half8{1, 1, 1, 1, 1, 1, 1, 1};

      // Tile loads.  Lane `lane` of load i moves logical chunk (lane % CPR) ^ swizzle
      // of row i * RPI + lane / CPR of this wave's rows into the LDS slot it writes.
      const int64_t head_bytes = static_cast<int64_t>(B) * ROWB;               // one (block, KV head)
      const int64_t block_bytes = static_cast<int64_t>(p.num_kv_heads) * head_bytes;
      const unsigned char* kmem = reinterpret_cast<const unsigned char*>(p.k_cache) + kvh * head_bytes;
      const unsigned char* vmem = reinterpret_cast<const unsigned char*>(p.v_cache) + kvh * head_bytes;
      unsigned voff[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rl = i * RPI + lane / CPR;
        voff[i] = rl * ROWB + ((lane % CPR) ^ lds_swizzle<D>(wave * RPW + rl)) * 16;
      }
      // Tiles are loaded by the waves in their softmax phase: K tiles by waves
      // 4-7, V tiles by waves 0-3.  Wave w moves row groups w mod 4 and
      // w mod 4 + 4 (rows 8 g .. 8 g + 7 of a tile, inside one block), with the
      // same lane offsets for both (the swizzle depends on the row mod 16 and
      // the groups are 32 rows apart).
      // Table entry of the block holding group g of tile jt, or 0 for rows past
      // t_end (tok < t_end <= cap: inside the table).  Read one phase pair before
      // the tile's load needs it, so that its latency never stalls a phase.
      auto block_of = [&](int jt, int g) __attribute__((always_inline)) {
        const int tok = jt * KT + g * RPW;
        return tok < t_end ? table[tok / B] : 0;
      };
      auto load_group = [&](const unsigned char* mem, unsigned char* dst, int jt, int g, int entry)
          __attribute__((always_inline)) {
        const int tok = jt * KT + g * RPW;   // the group's first row
        const int rows = max(0, min(RPW, t_end - tok));
        // The same id in every lane: kept in a scalar register, so the buffer
        // resource is one too.
        const int raw = __builtin_amdgcn_readfirstlane(entry);
        const bool ok = rows > 0 && static_cast<unsigned>(raw) < static_cast<unsigned>(p.num_blocks);
        load_rows(mem + (ok ? raw : 0) * block_bytes + (tok % B) * ROWB, ok ? rows * ROWB : 0,
                  dst + g * RPW * ROWB, voff[0], voff[NI - 1], NI);
      };
      const int g0 = wave % (NW / 2), g1 = g0 + NW / 2;   // this wave's row groups
      auto load_tile = [&](const unsigned char* mem, unsigned char* dst, int jt, const int (&e)[2])
          __attribute__((always_inline)) {
        load_group(mem, dst, jt, g0, e[0]);
        load_group(mem, dst, jt, g1, e[1]);
      };

      // Fragment addresses (bytes within a tile buffer).  K: row li of a 16-token
      // step, chunk grp + 4 kk.  V: row 4 grp + li / 4 of a 16-token step, bytes
      // 32 db + 8 (li % 4) of it.
      const int kswz = lds_swizzle<D>(li);
      const int vrow = 4 * grp + (li >> 2);
      const int vswz = lds_swizzle<D>(vrow);
      int koff[KSTEPS], vof[DBLK];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) koff[kk] = li * ROWB + ((grp + 4 * kk) ^ kswz) * 16;
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
        vof[db] = vrow * ROWB + ((2 * db + ((li >> 1) & 1)) ^ vswz) * 16 + 8 * (li & 1);

      float4_t s[NS][SUB];                     // scores of the tile last scored
      float4_t pa[NS][SUB];                    // its probabilities after the softmax phase (fp32)

      // Operand reads run ahead of the matrix instructions that use them: the
      // next step's fragments are issued before this step's MFMAs, and
      // scheduling barriers keep the compiler from pulling the reads back, so a
      // step never waits for the full LDS latency of its own reads.
      auto scores = [&](const unsigned char* kb) __attribute__((always_inline)) {
        half8 kf[2][KSTEPS];                   // K fragments of two 16-token steps
        auto ldk = [&](int sub, half8 (&dst)[KSTEPS]) __attribute__((always_inline)) {
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk)
            dst[kk] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(kb + sub * 16 * ROWB + koff[kk]));
        };
        ldk(0, kf[0]);
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub) {
          if (sub + 1 < SUB) ldk(sub + 1, kf[(sub + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int cs = 0; cs < NS; ++cs) s[cs][sub] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
            for (int cs = 0; cs < NS; ++cs)
              s[cs][sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[sub & 1][kk], qb[cs][kk], s[cs][sub], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // P.V over 32 tokens per MFMA (the double-rate 16x16x32 form): slots 0-3 of a
      // lane's operand are tokens 4*grp..4*grp+3 of one 16-token step, slots 4-7
      // the same rows of the next step, in A (probabilities) and B (transposed V)
      // alike, so the sum over k pairs each probability with its own V row.
      // The V operands of step i (32 tokens, 16 dimensions: two transposed reads)
      // are read kPvAhead steps before step i's MFMAs, into a ring of
      // kPvAhead + 1 operands.
      auto pv = [&](const unsigned char* vb) __attribute__((always_inline)) {
        constexpr int NSTEP = (SUB / 2) * DBLK;
        constexpr int AHEAD = kPvAhead;
        half8 vr[AHEAD + 1];
        auto ldv = [&](int i, half8& dst) __attribute__((always_inline)) {
          const unsigned char* src = vb + 2 * (i / DBLK) * 16 * ROWB + vof[i % DBLK];
          const half4 v0 = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)src));
          const half4 v1 =
              __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(src + 16 * ROWB)));
          dst = half8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        };
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) ldv(i, vr[i]);
        half8 pa8[NS];
#pragma unroll
        for (int i = 0; i < NSTEP; ++i) {
          if (i + AHEAD < NSTEP) ldv(i + AHEAD, vr[(i + AHEAD) % (AHEAD + 1)]);
          __builtin_amdgcn_sched_barrier(0);
          const int sp = 2 * (i / DBLK), db = i % DBLK;
          if (db == 0) {
#pragma unroll
            for (int cs = 0; cs < NS; ++cs) {
              pa8[cs] = half8{static_cast<_Float16>(pa[cs][sp][0]), static_cast<_Float16>(pa[cs][sp][1]),
                              static_cast<_Float16>(pa[cs][sp][2]), static_cast<_Float16>(pa[cs][sp][3]),
                              static_cast<_Float16>(pa[cs][sp + 1][0]), static_cast<_Float16>(pa[cs][sp + 1][1]),
                              static_cast<_Float16>(pa[cs][sp + 1][2]), static_cast<_Float16>(pa[cs][sp + 1][3])};
              den[cs] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa8[cs], ones, den[cs], 0, 0, 0);
            }
          }
#pragma unroll
          for (int cs = 0; cs < NS; ++cs)
            o[cs][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa8[cs], vr[i % (AHEAD + 1)], o[cs][db], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // Softmax phase of tile jt: per set one maximum over the tile, then the
      // probabilities relative to the running maximum, which moves only when the
      // tile's maximum exceeds it by more than kSlack (log2 units); then o and
      // den are rescaled once.
      auto softmax = [&](int jt) __attribute__((always_inline)) {
        const int tok0 = jt * KT;
        if (tok0 + KT - 1 > wave_pos_min) {    // some column sees only part of the tile
#pragma unroll
          for (int cs = 0; cs < NS; ++cs)
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int t = tok0 + sub * 16 + 4 * grp + r;
                s[cs][sub][r] = t <= pos[cs] ? s[cs][sub][r] : -INFINITY;
              }
        }
#pragma unroll
        for (int cs = 0; cs < NS; ++cs) {
          // Maximum of the raw scores (the scale is positive), then in log2 units.
          float mt = -INFINITY;
#pragma unroll
          for (int sub = 0; sub < SUB; ++sub)
            mt = fmaxf(mt, fmaxf(fmaxf(s[cs][sub][0], s[cs][sub][1]), fmaxf(s[cs][sub][2], s[cs][sub][3])));
          mt = column_max(mt) * p.scale_log2;
          const bool moved = mt > m[cs] + kSlack;
          const float m_new = moved ? mt : m[cs];
#pragma unroll
          for (int sub = 0; sub < SUB; ++sub) {
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(fmaf(s[cs][sub][r], p.scale_log2, -m_new));
            pa[cs][sub] = float4_t{pr[0], pr[1], pr[2], pr[3]};
          }
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
          m[cs] = m_new;
        }
      };
      // Matrix phase j: P.V of tile j - 1, then the scores of tile j.
      auto matrix_phase = [&](int j, const unsigned char* kb, const unsigned char* vb_prev)
          __attribute__((always_inline)) {
        if (j >= 1 && j - 1 <= last) pv(vb_prev);
        if (j < n && j <= last) scores(kb);
      };
      auto softmax_phase = [&](int j) __attribute__((always_inline)) {
        if (j >= 0 && j <= last) softmax(j);
      };
      // Phases 2mm and 2mm + 1.  K(j) lives in buffer j % 2 of kt*, V(j) of vt*.
      // Pair mm loads K(mm+1) (waves 4-7, at the start of phase 2mm) and V(mm)
      // (waves 0-3, at the start of phase 2mm + 1); both are waited for before
      // the barrier that ends phase 2mm + 1.  entry: the loading wave's table
      // entries (groups g0, g1) for the tile it loads in this pair, read one
      // pair ahead.
      PairClock pc;                            // empty unless built with PKV_WAVE_TIMELINE
      constexpr int kAhead = XO ? 1 : 0;      // tile loaded in pair mm: mm + kAhead
      int entry[2] = {block_of(kAhead, g0), block_of(kAhead, g1)};
      auto phase_pair = [&](int mm, unsigned char* kc, unsigned char* kn, unsigned char* vc,
                            const unsigned char* vp) __attribute__((always_inline)) {
        int entry_after[2] = {0, 0};
        pc.mark(0);
        if constexpr (XO) {
          if (mm + 1 < n) load_tile(kmem, kn, mm + 1, entry);
          pc.mark(1);
          entry_after[0] = block_of(mm + 2, g0);   // lands by the wait that ends this pair
          entry_after[1] = block_of(mm + 2, g1);
          softmax_phase(mm - 1);
        } else {
          pc.mark(1);
          matrix_phase(mm, kc, vp);
        }
        pc.mark(2);
        // No barrier between the halves: nothing one group writes in this pair is
        // read by the other in it (the loads go to the buffers the previous pair
        // finished with), and the barrier below starts every pair together.
        pc.mark(3);
        if constexpr (XO) {
          pc.mark(4);
          matrix_phase(mm, kc, vp);
        } else {
          if (mm < n) load_tile(vmem, vc, mm, entry);
          pc.mark(4);
          entry_after[0] = block_of(mm + 1, g0);
          entry_after[1] = block_of(mm + 1, g1);
          softmax_phase(mm);
        }
        pc.mark(5);
        __builtin_amdgcn_s_waitcnt(kWaitVmem);   // this wave's tile loads have landed
        pc.mark(6);
        __syncthreads();                          // and everyone's: K(mm+1), V(mm) readable
        pc.end_pair(mm);
        entry[0] = entry_after[0];
        entry[1] = entry_after[1];
      };

      if constexpr (XO) {
        const int e0[2] = {block_of(0, g0), block_of(0, g1)};
        load_tile(kmem, kt0, 0, e0);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmem);
      __syncthreads();
      for (int mm = 0; mm <= n; mm += 2) {
        phase_pair(mm, kt0, kt1, vt0, vt1);
        if (mm + 1 > n) break;
        phase_pair(mm + 1, kt1, kt0, vt1, vt0);
      }
      pc.finish(k, wave, j0 + NW * QW <= nq);
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
  };
  if (wave >= NW / 2)
    run(std::true_type{});
  else
    run(std::false_type{});
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

namespace pkv_decode {
hipError_t wave_timeline_read_prefill(void* dst, size_t bytes, bool clear) {
  return prefill_timeline_copy(dst, bytes, clear);
}
}  // namespace pkv_decode

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
  // Cost of a block = tokens its workgroup reads = position of its last query + 1.
  // Requests in order of their largest block, most first; each request's blocks
  // consecutive, most first.
  struct Key {
    int64_t req_cost, cost;
    int32_t s, b;
  };
  std::vector<Key> keys;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t nq = q_lens[s] > 0 ? q_lens[s] : 0;
    const int64_t len = context_lens[s] > 0 ? context_lens[s] : 0;
    const int64_t nblocks = (nq + qb - 1) / qb;
    if (nblocks > 65536)
      return fail(PKV_ERR_INVALID_ARG, "pa_prefill_plan: request %d has too many query blocks", s);
    const size_t first = keys.size();
    int64_t req_cost = 0;
    for (int64_t b = 0; b < nblocks; ++b) {
      const int64_t last = std::min<int64_t>((b + 1) * qb, nq) - 1;
      int64_t cost = len - nq + last + 1;
      cost = cost < 0 ? 0 : (cost > len ? len : cost);
      req_cost = std::max(req_cost, cost);
      keys.push_back(Key{0, cost, s, static_cast<int32_t>(b)});
    }
    for (size_t i = first; i < keys.size(); ++i) keys[i].req_cost = req_cost;
  }
  *num_items_out = static_cast<int32_t>(keys.size());
  if (static_cast<int64_t>(keys.size()) > items_capacity)
    return fail(PKV_ERR_INVALID_ARG, "pa_prefill_plan: %zu items do not fit in %d", keys.size(),
                items_capacity);
  if (!keys.empty() && !items) return fail(PKV_ERR_INVALID_ARG, "pa_prefill_plan: NULL items");
  std::sort(keys.begin(), keys.end(), [](const Key& a, const Key& b) {
    if (a.req_cost != b.req_cost) return a.req_cost > b.req_cost;
    if (a.s != b.s) return a.s < b.s;
    if (a.cost != b.cost) return a.cost > b.cost;
    return a.b < b.b;
  });
  for (size_t i = 0; i < keys.size(); ++i)
    items[i] = (static_cast<uint32_t>(keys[i].s) << 16) | static_cast<uint32_t>(keys[i].b);
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
