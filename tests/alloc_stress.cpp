// Stress driver for the host block allocator, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_allocator_sanitized.py (host code
// only; no device code is involved).  Random create / fork / append / batch
// append / free / bad-id operations; after every operation the invariants that
// the C ABI exposes are checked:
//   free + used == num_blocks; sum of table lengths == sum of refcounts;
//   distinct blocks over all tables == used; each table holds ceil(len/B)
//   blocks; lengths match the driver's own count; a failed call changes
//   nothing; after freeing everything all blocks are free again.
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
    std::vector<int32_t> live;
    std::vector<int64_t> len;          // by id
    std::vector<int64_t> slots(4096);
    std::vector<int32_t> pairs(2 * 4096);
    int64_t epoch = 0;
    for (int it = 0; it < iters / 8; ++it) {
      kv_stats before{};
      CHECK(kv_allocator_stats(a, &before) == PKV_OK);
      const int op = static_cast<int>(rng() % 7);
      int rc = PKV_OK;
      if (op == 0 || live.empty()) {
        int32_t s = -1;
        CHECK(kv_seq_create(a, &s) == PKV_OK);
        if (static_cast<size_t>(s) >= len.size()) len.resize(s + 1, 0);
        len[s] = 0;
        live.push_back(s);
      } else if (op == 1) {
        int32_t p = live[rng() % live.size()], c = -1;
        CHECK(kv_seq_fork(a, p, &c) == PKV_OK);
        if (static_cast<size_t>(c) >= len.size()) len.resize(c + 1, 0);
        len[c] = len[p];
        live.push_back(c);
      } else if (op == 2) {
        int32_t s = live[rng() % live.size()];
        int32_t n = static_cast<int32_t>(rng() % (3 * bs + 1));
        int32_t pair[2], ncow = 0;
        rc = kv_seq_append(a, s, n, slots.data(), pair, &ncow);
        if (rc == PKV_OK) {
          len[s] += n;
          CHECK(ncow == 0 || ncow == 1);
        }
      } else if (op == 3) {
        std::vector<int32_t> batch;
        const size_t k = 1 + rng() % (2 * live.size());
        for (size_t i = 0; i < k && i < 4096; ++i) batch.push_back(live[rng() % live.size()]);
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
          rc = kv_decode_step_host(a, batch.data(), n, 0, -1, 8, 2, 64, PKV_F16, part, 0, nullptr,
                                   0, &lay);
          CHECK(rc == PKV_ERR_INVALID_ARG && lay.total_bytes > 0);
          std::vector<char> buf(lay.total_bytes);
          rc = kv_decode_step_host(a, batch.data(), n, 0, -1, 8, 2, 64, PKV_F16, part, 0,
                                   buf.data(), buf.size(), &lay);
          if (rc == PKV_OK) {
            ncow = lay.num_pairs;
            const int32_t* lens_out = reinterpret_cast<const int32_t*>(buf.data() + lay.lens_offset);
            std::map<int32_t, int64_t> want;
            for (int32_t s : batch) want[s] = (want.count(s) ? want[s] : len[s]) + 1;
            for (int32_t i = 0; i < n; ++i) CHECK(lens_out[i] == want[batch[i]]);
            CHECK(lay.plan.num_items >= 1 && lay.items_offset + 4ull * lay.plan.num_items <= buf.size());
          }
        }
        if (rc == PKV_OK) {
          for (int32_t s : batch) len[s] += 1;
          CHECK(ncow >= 0 && ncow <= static_cast<int32_t>(batch.size()));
        }
      } else if (op == 4) {
        const size_t i = rng() % live.size();
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
      } else {
        int32_t s = live[rng() % live.size()];
        int32_t pair[2], ncow = 0;
        rc = kv_seq_append(a, s, nb * bs + 1, slots.data(), pair, &ncow);   // never fits
        CHECK(rc == PKV_ERR_OUT_OF_BLOCKS);
      }
      kv_stats st{};
      CHECK(kv_allocator_stats(a, &st) == PKV_OK);
      if (rc != PKV_OK) {                     // all or nothing
        CHECK(rc == PKV_ERR_OUT_OF_BLOCKS);
        CHECK(st.free_blocks == before.free_blocks && st.sum_refcounts == before.sum_refcounts &&
              st.live_tokens == before.live_tokens);
      }
      CHECK(st.free_blocks + st.used_blocks + st.pending_blocks == nb);
      CHECK(st.shared_blocks <= st.used_blocks);
      if (!live.empty()) {
        const int32_t maxb = nb;
        std::vector<int32_t> tables(static_cast<size_t>(live.size()) * maxb), lens(live.size());
        CHECK(kv_export_block_tables(a, live.data(), static_cast<int32_t>(live.size()), maxb, -1,
                                     tables.data(), lens.data()) == PKV_OK);
        std::vector<int32_t> lens2(live.size());
        CHECK(kv_seq_lens(a, live.data(), static_cast<int32_t>(live.size()), lens2.data()) == PKV_OK);
        int64_t total = 0;
        std::set<int32_t> distinct;
        for (size_t i = 0; i < live.size(); ++i) {
          CHECK(lens[i] == len[live[i]] && lens2[i] == lens[i]);
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
    kv_allocator_destroy(a);
  }
  std::printf("ok\n");
  return 0;
}
