// Stress driver for the host block allocator, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_allocator_sanitized.py (host code
// only; no device code is involved).  Random create / fork / append / batch
// append / free / swap-out / swap-in / bad-id operations; after every
// operation the invariants that the C ABI exposes are checked:
//   free + used + parked == blocks, for the device pool and the host tier;
//   sum of resident table lengths == sum of refcounts; distinct blocks over the
//   resident tables == used; each table holds ceil(len/B) blocks; lengths match
//   the driver's own count; swapped sequences are refused by append, fork and
//   export; a failed call changes nothing; after freeing everything all blocks
//   of both tiers are free again.  Swap pair lists go into heap buffers of
//   exactly the size the call asks for, so a write past the end is caught.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <map>
#include <set>
#include <vector>

#include "pagedkv.h"

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);      \
      std::exit(1);                                                           \
    }                                                                         \
  } while (0)

// Prefix groups of one step (kv_decode_step_host with PKV_STEP_GROUPS): every
// token of every request is computed exactly once, by a group piece or by the
// request's own piece; tokens a group covers lie in the same physical blocks
// of all its members' tables and within their lengths.
static long g_grouped_steps = 0;

static void check_groups(const char* base, const kv_step_layout& lay, int32_t n, int32_t bs) {
  g_grouped_steps += lay.num_groups > 0;
  const int32_t* tables = reinterpret_cast<const int32_t*>(base + lay.tables_offset);
  const int32_t* lens = reinterpret_cast<const int32_t*>(base + lay.lens_offset);
  const uint32_t* items = reinterpret_cast<const uint32_t*>(base + lay.items_offset);
  const int32_t* groups = reinterpret_cast<const int32_t*>(base + lay.groups_offset);
  const uint32_t* gitems = reinterpret_cast<const uint32_t*>(base + lay.group_items_offset);
  const int32_t* shared =
      lay.num_groups > 0 ? reinterpret_cast<const int32_t*>(base + lay.shared_lens_offset) : nullptr;
  const int32_t pt = lay.plan.partition_size;
  const int32_t w = lay.max_blocks;
  std::vector<std::vector<int>> count(static_cast<size_t>(n));
  for (int32_t s = 0; s < n; ++s) count[s].assign(static_cast<size_t>(lens[s]), 0);
  for (int32_t i = 0; i < lay.plan.num_items; ++i) {
    const int32_t s = static_cast<int32_t>(items[i] >> 16), p = static_cast<int32_t>(items[i] & 0xFFFF);
    CHECK(s < n);
    int64_t lo = pt > 0 ? static_cast<int64_t>(p) * pt : 0;
    const int64_t hi = pt > 0 ? std::min<int64_t>(lo + pt, lens[s]) : lens[s];
    if (shared && shared[s] > lo && shared[s] < lo + pt) lo = shared[s];
    CHECK(lo < hi || lens[s] == 0);
    for (int64_t t = lo; t < hi; ++t) count[s][t] += 1;
  }
  if (lay.num_group_items > 0) CHECK(pt > 0 && pt % bs == 0);
  for (int32_t g = 0; g < lay.num_groups; ++g) {
    const int32_t* row = groups + static_cast<int64_t>(g) * PKV_GROUP_STRIDE;
    CHECK(row[0] >= 2 && row[0] <= 4);         // 8 query heads over 2 KV heads: 16 / 4 members
    std::set<int32_t> mem(row + 1, row + 1 + row[0]);
    CHECK(static_cast<int32_t>(mem.size()) == row[0]);
    for (int32_t m : mem) CHECK(m >= 0 && m < n && shared[m] == shared[row[1]]);
  }
  for (int32_t k = 0; k < lay.num_group_items; ++k) {
    const int32_t g = static_cast<int32_t>(gitems[k] >> 16), p = static_cast<int32_t>(gitems[k] & 0xFFFF);
    CHECK(g < lay.num_groups);
    const int32_t* row = groups + static_cast<int64_t>(g) * PKV_GROUP_STRIDE;
    const int32_t first = row[1];
    const int64_t lo = static_cast<int64_t>(p) * pt;
    int64_t hi = lo + pt;
    if (shared[first] > lo && shared[first] < hi) hi = shared[first];
    for (int32_t j = 0; j < row[0]; ++j) {
      const int32_t m = row[1 + j];
      CHECK(hi <= lens[m]);
      for (int64_t b = lo / bs; b < (hi + bs - 1) / bs; ++b)
        CHECK(b < w && tables[static_cast<int64_t>(m) * w + b] == tables[static_cast<int64_t>(first) * w + b]);
      for (int64_t t = lo; t < hi; ++t) count[m][t] += 1;
    }
  }
  for (int32_t s = 0; s < n; ++s)
    for (int c : count[s]) CHECK(c == 1);
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  std::mt19937 rng(7);
  for (int trial = 0; trial < 8; ++trial) {
    const int32_t nb = 8 + static_cast<int32_t>(rng() % 120);
    const int32_t bs = 1 << (rng() % 5);
    std::vector<int32_t> order(nb);
    for (int32_t i = 0; i < nb; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    kv_allocator* a = nullptr;
    CHECK(kv_allocator_create(nb, bs, order.data(), &a) == PKV_OK);
    const int32_t nh = 4 + static_cast<int32_t>(rng() % 100);
    CHECK(kv_allocator_add_host_tier(a, nh, nullptr) == PKV_OK);
    CHECK(kv_allocator_add_host_tier(a, nh, nullptr) == PKV_ERR_INVALID_ARG);
    std::vector<int32_t> live;
    std::set<int32_t> swapped;
    std::vector<int64_t> len;          // by id
    std::vector<int64_t> slots(4096);
    std::vector<int32_t> pairs(2 * 4096);
    int64_t epoch = 0;
    for (int it = 0; it < iters / 8; ++it) {
      kv_stats before{};
      CHECK(kv_allocator_stats(a, &before) == PKV_OK);
      const int op = static_cast<int>(rng() % 9);
      int rc = PKV_OK;
      std::vector<int32_t> resident;
      for (int32_t s : live)
        if (!swapped.count(s)) resident.push_back(s);
      if (op == 0 || live.empty() || (op <= 3 && resident.empty())) {
        int32_t s = -1;
        CHECK(kv_seq_create(a, &s) == PKV_OK);
        if (static_cast<size_t>(s) >= len.size()) len.resize(s + 1, 0);
        len[s] = 0;
        live.push_back(s);
      } else if (op == 1) {
        int32_t p = resident[rng() % resident.size()], c = -1;
        CHECK(kv_seq_fork(a, p, &c) == PKV_OK);
        if (static_cast<size_t>(c) >= len.size()) len.resize(c + 1, 0);
        len[c] = len[p];
        live.push_back(c);
      } else if (op == 2) {
        int32_t s = resident[rng() % resident.size()];
        int32_t n = static_cast<int32_t>(rng() % (3 * bs + 1));
        int32_t pair[2], ncow = 0;
        rc = kv_seq_append(a, s, n, slots.data(), pair, &ncow);
        if (rc == PKV_OK) {
          len[s] += n;
          CHECK(ncow == 0 || ncow == 1);
        }
      } else if (op == 3) {
        std::vector<int32_t> batch;
        const size_t k = 1 + rng() % (2 * resident.size());
        for (size_t i = 0; i < k && i < 4096; ++i) batch.push_back(resident[rng() % resident.size()]);
        int32_t ncow = 0;
        if (rng() % 2) {
          rc = kv_batch_append(a, batch.data(), static_cast<int32_t>(batch.size()), slots.data(),
                               pairs.data(), &ncow);
        } else {
          // The fused step call into a heap buffer of exactly the size it asks for,
          // so a write past its end is caught by the sanitizer.
          kv_step_layout lay{};
          const int32_t n = static_cast<int32_t>(batch.size());
          const int32_t part = static_cast<int32_t>(rng() % 3) == 0 ? -1 : bs * (1 + rng() % 4);
          const int32_t flags = rng() % 2 ? PKV_STEP_GROUPS : 0;
          rc = kv_decode_step_host(a, batch.data(), n, 0, -1, 8, 2, 64, PKV_F16, part, 0, flags,
                                   nullptr, 0, &lay);
          CHECK(rc == PKV_ERR_INVALID_ARG && lay.total_bytes > 0);
          std::vector<char> buf(lay.total_bytes);
          rc = kv_decode_step_host(a, batch.data(), n, 0, -1, 8, 2, 64, PKV_F16, part, 0, flags,
                                   buf.data(), buf.size(), &lay);
          if (rc == PKV_OK) {
            ncow = lay.num_pairs;
            const int32_t* lens_out = reinterpret_cast<const int32_t*>(buf.data() + lay.lens_offset);
            std::map<int32_t, int64_t> want;
            for (int32_t s : batch) want[s] = (want.count(s) ? want[s] : len[s]) + 1;
            for (int32_t i = 0; i < n; ++i) CHECK(lens_out[i] == want[batch[i]]);
            CHECK(lay.plan.num_items + lay.num_group_items >= 1 &&
                  lay.items_offset + 4ull * lay.plan.num_items <= buf.size());
            CHECK(flags || lay.num_groups == 0);
            CHECK(lay.group_items_offset + 4ull * lay.num_group_items <= buf.size());
            check_groups(buf.data(), lay, n, bs);
          }
        }
        if (rc == PKV_OK) {
          for (int32_t s : batch) len[s] += 1;
          CHECK(ncow >= 0 && ncow <= static_cast<int32_t>(batch.size()));
        }
      } else if (op == 4) {
        const size_t i = rng() % live.size();
        swapped.erase(live[i]);
        if (rng() % 2) {
          CHECK(kv_seq_free(a, live[i]) == PKV_OK);
        } else {
          epoch += static_cast<int64_t>(rng() % 2);
          CHECK(kv_seq_free_deferred(a, live[i], epoch) == PKV_OK);
          int32_t released = -1;
          CHECK(kv_allocator_retire(a, epoch - static_cast<int64_t>(rng() % 3), &released) == PKV_OK);
          CHECK(released >= 0);
        }
        live.erase(live.begin() + static_cast<long>(i));
      } else if (op == 5) {
        int32_t l = 0, pair[2], ncow = 0;
        const int32_t bad = static_cast<int32_t>(rng() % 3) == 0 ? -5 : 1 << 30;
        CHECK(kv_seq_len(a, bad, &l) == PKV_ERR_BAD_SEQ);
        CHECK(kv_seq_append(a, bad, 1, slots.data(), pair, &ncow) == PKV_ERR_BAD_SEQ);
        CHECK(kv_seq_free(a, bad) == PKV_ERR_BAD_SEQ);
      } else if (op == 6) {
        if (resident.empty()) continue;
        int32_t s = resident[rng() % resident.size()];
        int32_t pair[2], ncow = 0;
        rc = kv_seq_append(a, s, nb * bs + 1, slots.data(), pair, &ncow);   // never fits
        CHECK(rc == PKV_ERR_OUT_OF_BLOCKS);
      } else if (op == 7) {
        // Swap a random distinct subset out (of the resident) or in (of the swapped).
        const bool out = swapped.empty() || (!resident.empty() && rng() % 2);
        std::vector<int32_t> from = out ? resident : std::vector<int32_t>(swapped.begin(), swapped.end());
        std::shuffle(from.begin(), from.end(), rng);
        from.resize(1 + rng() % from.size());
        const int32_t n = static_cast<int32_t>(from.size());
        const int32_t deferred = static_cast<int32_t>(rng() % 2);
        epoch += deferred;
        auto call = out ? kv_swap_out : kv_swap_in;
        int32_t need = 0;
        rc = call(a, from.data(), n, deferred, epoch, nullptr, 0, &need);
        if (rc == PKV_ERR_INVALID_ARG) {
          CHECK(need > 0);
          std::vector<int32_t> exact(2 * static_cast<size_t>(need));
          int32_t got = 0;
          if (need > 1) {
            CHECK(call(a, from.data(), n, deferred, epoch, exact.data(), need - 1, &got) ==
                  PKV_ERR_INVALID_ARG && got == need);
          }
          rc = call(a, from.data(), n, deferred, epoch, exact.data(), need, &got);
          if (rc == PKV_OK) {
            CHECK(got == need);
            std::set<int32_t> news;
            for (int32_t j = 0; j < got; ++j) {
              CHECK(exact[2 * j] >= 0 && exact[2 * j] < (out ? nb : nh));
              CHECK(exact[2 * j + 1] >= 0 && exact[2 * j + 1] < (out ? nh : nb));
              news.insert(exact[2 * j + 1]);
            }
            CHECK(static_cast<int32_t>(news.size()) == got);
          }
        } else {
          CHECK(rc == PKV_OK && need == 0);   // nothing to copy (empty sequences)
        }
        if (rc == PKV_OK) {
          for (int32_t s : from) {
            if (out) swapped.insert(s); else swapped.erase(s);
          }
          int32_t released = -1;
          CHECK(kv_allocator_retire(a, epoch - static_cast<int64_t>(rng() % 2), &released) == PKV_OK);
          CHECK(released >= 0);
        } else {
          CHECK(rc == PKV_ERR_OUT_OF_BLOCKS);
        }
      } else {
        // Refusals: a swapped sequence cannot grow, fork or be exported; a resident
        // one cannot be swapped in; a set may not list a sequence twice.
        if (!swapped.empty()) {
          const int32_t s = *swapped.begin();
          int32_t pair[2], ncow = 0, c = -1, flag = 0, np = 0;
          CHECK(kv_seq_append(a, s, 1, slots.data(), pair, &ncow) == PKV_ERR_SWAPPED);
          CHECK(kv_seq_fork(a, s, &c) == PKV_ERR_SWAPPED);
          std::vector<int32_t> t(nb);
          int32_t l = 0;
          CHECK(kv_export_block_tables(a, &s, 1, nb, -1, t.data(), &l) == PKV_ERR_SWAPPED);
          CHECK(kv_seq_is_swapped(a, s, &flag) == PKV_OK && flag == 1);
          CHECK(kv_swap_out(a, &s, 1, 0, 0, pairs.data(), 4096, &np) == PKV_ERR_SWAPPED);
        }
        if (!resident.empty()) {
          int32_t two[2] = {resident[0], resident[0]}, np = 0;
          CHECK(kv_swap_in(a, two, 1, 0, 0, pairs.data(), 4096, &np) == PKV_ERR_SWAPPED);
          CHECK(kv_swap_out(a, two, 2, 0, 0, pairs.data(), 4096, &np) == PKV_ERR_INVALID_ARG);
        }
      }
      kv_stats st{};
      CHECK(kv_allocator_stats(a, &st) == PKV_OK);
      if (rc != PKV_OK) {                     // all or nothing
        CHECK(rc == PKV_ERR_OUT_OF_BLOCKS);
        CHECK(st.free_blocks == before.free_blocks && st.sum_refcounts == before.sum_refcounts &&
              st.live_tokens == before.live_tokens &&
              st.host_free_blocks == before.host_free_blocks &&
              st.swapped_seqs == before.swapped_seqs);
      }
      CHECK(st.free_blocks + st.used_blocks + st.pending_blocks == nb);
      CHECK(st.host_free_blocks + st.host_used_blocks + st.host_pending_blocks == nh);
      CHECK(st.host_blocks == nh && st.swapped_seqs == static_cast<int32_t>(swapped.size()));
      CHECK(st.shared_blocks <= st.used_blocks);
      resident.clear();
      for (int32_t s : live)
        if (!swapped.count(s)) resident.push_back(s);
      if (!resident.empty()) {
        const int32_t maxb = nb;
        std::vector<int32_t> tables(static_cast<size_t>(resident.size()) * maxb),
            lens(resident.size());
        CHECK(kv_export_block_tables(a, resident.data(), static_cast<int32_t>(resident.size()),
                                     maxb, -1, tables.data(), lens.data()) == PKV_OK);
        std::vector<int32_t> lens2(resident.size());
        CHECK(kv_seq_lens(a, resident.data(), static_cast<int32_t>(resident.size()),
                          lens2.data()) == PKV_OK);
        int64_t total = 0;
        std::set<int32_t> distinct;
        for (size_t i = 0; i < resident.size(); ++i) {
          CHECK(lens[i] == len[resident[i]] && lens2[i] == lens[i]);
          int64_t held = 0;
          for (int32_t j = 0; j < maxb; ++j) {
            const int32_t b = tables[i * maxb + j];
            if (b < 0) break;
            CHECK(b < nb);
            distinct.insert(b);
            ++held;
          }
          CHECK(held == (lens[i] + bs - 1) / bs);
          total += held;
        }
        CHECK(total == st.sum_refcounts);
        CHECK(static_cast<int32_t>(distinct.size()) == st.used_blocks);
      }
    }
    for (int32_t s : live) CHECK(kv_seq_free(a, s) == PKV_OK);
    CHECK(kv_allocator_retire(a, epoch, nullptr) == PKV_OK);
    kv_stats st{};
    CHECK(kv_allocator_stats(a, &st) == PKV_OK);
    CHECK(st.free_blocks == nb && st.sum_refcounts == 0);
    CHECK(st.host_free_blocks == nh && st.swapped_seqs == 0);
    kv_allocator_destroy(a);
  }
  std::printf("ok grouped_steps=%ld\n", g_grouped_steps);
  return 0;
}
