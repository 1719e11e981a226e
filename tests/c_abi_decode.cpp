// One decode step driven through the C ABI of libpagedkv.so alone: no Python,
// no torch.  The host allocator reserves slots (with a fork whose append
// copies the shared, partly filled last block), kv_copy_blocks and
// kv_cache_write fill the pools, and pa_decode attends, on one stream.
//
// Checks are exact properties of attention ("Only 20.4% of your KV cache held
// actual tokens" (blog.teqners.com), section "The page table, relocated into
// attention"; "The part everyone forgets: pages enable sharing, not just
// packing"):
//   * written and copied K/V bytes read back bit for bit; the copy-on-write
//     source block keeps the other reader's tokens;
//   * a one-token context returns that token's V exactly;
//   * keys that are all equal give equal weights, so the output is the mean of
//     the context's V (within 1e-5 relative);
// for a single pass and for 16-token partitions with the reduce.
// Prints "c_abi_decode OK" and exits 0 on success.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "pagedkv.h"

#define HIP_CHECK(x)                                                             \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      return 1;                                                                  \
    }                                                                            \
  } while (0)
#define PKV_CHECK(x)                                                             \
  do {                                                                           \
    if ((x) != PKV_OK) {                                                         \
      std::fprintf(stderr, "%s: %s\n", #x, pkv_last_error());                    \
      return 1;                                                                  \
    }                                                                            \
  } while (0)
#define EXPECT(c)                                                                \
  do {                                                                           \
    if (!(c)) {                                                                  \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);          \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

namespace {

constexpr int NB = 32, HKV = 2, HQ = 4, D = 64, B = 16;
constexpr int ROW = HKV * D;                     // halves per token row of k_new / v_new

using half = _Float16;

// Pool index of (block, KV head, slot in block, dim).
size_t at(int blk, int h, int slot, int d) {
  return ((static_cast<size_t>(blk) * HKV + h) * B + slot) * D + d;
}

}  // namespace

int main() {
  std::mt19937 rng(11);
  std::uniform_int_distribution<int> small(-8, 8);
  auto rand_half = [&] { return static_cast<half>(small(rng) * 0.125f); };   // exact in fp16

  // --- allocator: seq a (1 token), seq b (40 tokens), c = fork(b) + 1 token.
  kv_allocator* al = nullptr;
  PKV_CHECK(kv_allocator_create(NB, B, nullptr, &al));
  int32_t a, b, c, ncow = 0, pair[2] = {-1, -1};
  std::vector<int64_t> slots_a(1), slots_b(40), slots_c(1);
  PKV_CHECK(kv_seq_create(al, &a));
  PKV_CHECK(kv_seq_append(al, a, 1, slots_a.data(), pair, &ncow));
  EXPECT(ncow == 0);
  PKV_CHECK(kv_seq_create(al, &b));
  PKV_CHECK(kv_seq_append(al, b, 40, slots_b.data(), pair, &ncow));
  EXPECT(ncow == 0);
  PKV_CHECK(kv_seq_fork(al, b, &c));
  PKV_CHECK(kv_seq_append(al, c, 1, slots_c.data(), pair, &ncow));
  EXPECT(ncow == 1 && pair[0] == slots_b[39] / B && pair[1] == slots_c[0] / B);

  // --- host tokens: a's one token; b's 40 tokens share one key per KV head.
  std::vector<half> key(ROW), k_a(ROW), v_a(ROW), k_b(40 * ROW), v_b(40 * ROW), v_c(ROW);
  for (auto& x : key) x = rand_half();
  for (auto& x : k_a) x = rand_half();
  for (auto& x : v_a) x = rand_half();
  for (int t = 0; t < 40; ++t) std::memcpy(&k_b[t * ROW], key.data(), ROW * sizeof(half));
  for (auto& x : v_b) x = rand_half();
  for (auto& x : v_c) x = rand_half();

  hipStream_t st;
  HIP_CHECK(hipStreamCreate(&st));
  const size_t pool = static_cast<size_t>(NB) * HKV * B * D;
  half *kp, *vp, *dk, *dv;
  int64_t* dslots;
  HIP_CHECK(hipMalloc(&kp, pool * sizeof(half)));
  HIP_CHECK(hipMalloc(&vp, pool * sizeof(half)));
  HIP_CHECK(hipMemset(kp, 0, pool * sizeof(half)));
  HIP_CHECK(hipMemset(vp, 0, pool * sizeof(half)));
  HIP_CHECK(hipMalloc(&dk, 40 * ROW * sizeof(half)));
  HIP_CHECK(hipMalloc(&dv, 40 * ROW * sizeof(half)));
  HIP_CHECK(hipMalloc(&dslots, 40 * sizeof(int64_t)));
  auto write = [&](const std::vector<int64_t>& slots, const half* k, const half* v) -> int {
    const int n = static_cast<int>(slots.size());
    HIP_CHECK(hipMemcpy(dk, k, n * ROW * sizeof(half), hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dv, v, n * ROW * sizeof(half), hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dslots, slots.data(), n * sizeof(int64_t), hipMemcpyHostToDevice));
    PKV_CHECK(kv_cache_write(kp, vp, NB, dk, dv, dslots, n, HKV, D, B, st));
    HIP_CHECK(hipStreamSynchronize(st));
    return 0;
  };
  if (write(slots_a, k_a.data(), v_a.data()) || write(slots_b, k_b.data(), v_b.data())) return 1;
  // c's append copied b's last block first; then c's own token goes into the copy.
  int32_t* dpair;
  HIP_CHECK(hipMalloc(&dpair, 2 * sizeof(int32_t)));
  HIP_CHECK(hipMemcpy(dpair, pair, sizeof(pair), hipMemcpyHostToDevice));
  void* kl[1] = {kp};
  void* vl[1] = {vp};
  PKV_CHECK(kv_copy_blocks(kl, vl, 1, dpair, 1, NB, HKV, D, B, st));
  if (write(slots_c, key.data(), v_c.data())) return 1;

  // --- bytes: every written token, and the copy next to its untouched source.
  std::vector<half> hk(pool), hv(pool);
  HIP_CHECK(hipMemcpy(hk.data(), kp, pool * sizeof(half), hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(hv.data(), vp, pool * sizeof(half), hipMemcpyDeviceToHost));
  auto same_token = [&](int64_t slot, const half* k, const half* v) {
    for (int h = 0; h < HKV; ++h)
      for (int d = 0; d < D; ++d) {
        const size_t i = at(static_cast<int>(slot / B), h, static_cast<int>(slot % B), d);
        if (std::memcmp(&hk[i], &k[h * D + d], 2) || std::memcmp(&hv[i], &v[h * D + d], 2))
          return false;
      }
    return true;
  };
  EXPECT(same_token(slots_a[0], k_a.data(), v_a.data()));
  for (int t = 0; t < 40; ++t) EXPECT(same_token(slots_b[t], &k_b[t * ROW], &v_b[t * ROW]));
  EXPECT(same_token(slots_c[0], key.data(), v_c.data()));
  for (int t = 32; t < 40; ++t)          // c's copy of b's last block, slot by slot
    EXPECT(same_token(static_cast<int64_t>(pair[1]) * B + t % B, &k_b[t * ROW], &v_b[t * ROW]));
  EXPECT(slots_c[0] == static_cast<int64_t>(pair[1]) * B + 8);
  for (int h = 0; h < HKV; ++h)          // b's source block still has no token 40
    for (int d = 0; d < D; ++d) EXPECT(hk[at(pair[0], h, 8, d)] == static_cast<half>(0.f));

  // --- decode: tables and lengths from the allocator.
  const int32_t seqs[3] = {a, b, c};
  const int32_t width = 3;
  int32_t tables[3 * width], lens[3];
  PKV_CHECK(kv_export_block_tables(al, seqs, 3, width, NB, tables, lens));
  EXPECT(lens[0] == 1 && lens[1] == 40 && lens[2] == 41);
  int32_t *dtab, *dlen;
  float *dq, *dout;
  HIP_CHECK(hipMalloc(&dtab, sizeof(tables)));
  HIP_CHECK(hipMalloc(&dlen, sizeof(lens)));
  HIP_CHECK(hipMemcpy(dtab, tables, sizeof(tables), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(dlen, lens, sizeof(lens), hipMemcpyHostToDevice));
  std::vector<float> q(3 * HQ * D), out(3 * HQ * D);
  std::uniform_real_distribution<float> u(-1.f, 1.f);
  for (auto& x : q) x = u(rng);
  HIP_CHECK(hipMalloc(&dq, q.size() * sizeof(float)));
  HIP_CHECK(hipMalloc(&dout, out.size() * sizeof(float)));
  HIP_CHECK(hipMemcpy(dq, q.data(), q.size() * sizeof(float), hipMemcpyHostToDevice));
  const int G = HQ / HKV;
  for (int part : {0, 16}) {
    const size_t ws_bytes = pa_decode_workspace_size(3, HQ, D, 41, part);
    void* ws = nullptr;
    if (ws_bytes) HIP_CHECK(hipMalloc(&ws, ws_bytes));
    HIP_CHECK(hipMemset(dout, 0xFF, out.size() * sizeof(float)));     // NaN until written
    PKV_CHECK(pa_decode(dout, dq, PKV_F32, kp, vp, NB, dtab, width, dlen, 3, HQ, HKV, D, B,
                        1.f / std::sqrt(static_cast<float>(D)), 41, part, nullptr, 0, 0, ws,
                        ws_bytes, st));
    HIP_CHECK(hipStreamSynchronize(st));
    HIP_CHECK(hipMemcpy(out.data(), dout, out.size() * sizeof(float), hipMemcpyDeviceToHost));
    if (ws) HIP_CHECK(hipFree(ws));
    for (int h = 0; h < HQ; ++h) {
      const int g = h / G;
      for (int d = 0; d < D; ++d) {
        // a: one token, weight exactly 1.
        EXPECT(out[(0 * HQ + h) * D + d] == static_cast<float>(v_a[g * D + d]));
        // b and c: equal keys, so the mean of V.
        double mb = 0.0, mc = 0.0;
        for (int t = 0; t < 40; ++t) mb += static_cast<double>(v_b[t * ROW + g * D + d]);
        mc = (mb + static_cast<double>(v_c[g * D + d])) / 41.0;
        mb /= 40.0;
        EXPECT(std::fabs(out[(1 * HQ + h) * D + d] - mb) <= 1e-5 * (1.0 + std::fabs(mb)));
        EXPECT(std::fabs(out[(2 * HQ + h) * D + d] - mc) <= 1e-5 * (1.0 + std::fabs(mc)));
      }
    }
  }
  kv_allocator_destroy(al);
  HIP_CHECK(hipStreamDestroy(st));
  std::printf("c_abi_decode OK\n");
  return 0;
}
