// Host launch planning: kernel policy and choice, the planner pa_decode_plan
// (partition size, work list longest piece first, residency limit) and its
// size helpers.  Plain C++, no HIP.
//
// Why: decode reads every cached byte of every request once per step ("800
// kilobytes per token" (shashforge.dev), section "The old answer, imported
// honestly"; "The KV cache is a systems problem" (rsw.lol), section "Calculate
// bytes per token before choosing a batch"), so a launch lasts as long as its
// busiest compute unit; batches mix short and long contexts ("Only 20.4% of
// your KV cache held actual tokens" (blog.teqners.com), section "Why the KV
// cache is the thing that limits your batch").
#include "decode_plan.h"

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <utility>
#include <vector>

#include "errors.h"
#include "pagedkv.h"

namespace pkv_plan {
namespace {

using pkv::fail;

int head_tile(int group) {
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

// Kernel policy for head groups (see pa_decode_set_kernel_policy).  The first
// value comes from PKV_GQA_KERNEL=valu in the environment, if set.
std::atomic<int> g_policy{-1};

int kernel_policy() {
  int v = g_policy.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* env = std::getenv("PKV_GQA_KERNEL");
    const int init = (env != nullptr && std::strcmp(env, "valu") == 0) ? PKV_POLICY_VALU
                                                                       : PKV_POLICY_DEFAULT;
    g_policy.compare_exchange_strong(v, init);
    v = g_policy.load(std::memory_order_relaxed);
  }
  return v;
}

}  // namespace

KernelChoice choose_kernel(int32_t q_dtype, int group) {
  const bool mfma = q_dtype == PKV_F16 && group % 4 == 0 && kernel_policy() != PKV_POLICY_VALU;
  if (mfma) return {true, group % 16 == 0 ? 16 : (group % 8 == 0 ? 8 : 4)};
  return {false, head_tile(group)};
}

namespace {

// Partition size chosen by pa_decode_plan (see pagedkv.h): lens already clamped >= 0.
int32_t auto_partition(const int32_t* lens, int32_t n, int tiles, int cus, int32_t block_size) {
  int64_t total = 0;
  int32_t longest = 0;
  for (int32_t i = 0; i < n; ++i) {
    total += lens[i];
    longest = lens[i] > longest ? lens[i] : longest;
  }
  const int64_t simds = static_cast<int64_t>(cus) * 4;
  const double share = static_cast<double>(total) * tiles / static_cast<double>(simds);
  if (static_cast<int64_t>(n) * tiles >= simds && longest <= 1.25 * share) return 0;
  int32_t part = 256;
  for (int32_t cand : {2048, 1024, 512}) {
    if (cand <= share / 2) {
      part = cand;
      break;
    }
  }
  return (part + block_size - 1) / block_size * block_size;
}

// Residency limit (waves per CU) for a launch, measured on MI355X: the MFMA
// kernel runs best with 6 (of the 8 its registers allow; 5, 7 and 8 were
// slower on the GQA and long-context mixes); the VALU kernel gains from 4
// only when requests run in one pass and their lengths are skewed (all pieces
// are resident at once otherwise, so the dispatcher cannot balance them),
// and loses a few percent with any limit on even lengths.
int residency_limit(bool mfma, int32_t part, const int32_t* lens, int32_t n) {
  if (mfma) return kMfmaWavesPerCu;
  if (part != 0 || n == 0) return 0;
  int64_t total = 0, nonempty = 0;
  int32_t longest = 0;
  for (int32_t i = 0; i < n; ++i) {
    total += lens[i];
    nonempty += lens[i] > 0;
    longest = std::max(longest, lens[i]);
  }
  if (nonempty == 0) return 0;
  return longest * nonempty > 1.5 * static_cast<double>(total) ? kValuSkewedWavesPerCu : 0;
}

}  // namespace
}  // namespace pkv_plan

using pkv::fail;
using namespace pkv_plan;

extern "C" int pa_decode_set_kernel_policy(int32_t policy) {
  if (policy != PKV_POLICY_DEFAULT && policy != PKV_POLICY_VALU)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_set_kernel_policy: unknown policy %d", policy);
  const int previous = kernel_policy();
  g_policy.store(policy, std::memory_order_relaxed);
  return previous;
}

extern "C" size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                           int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return workspace_bytes_for(num_seqs, num_q_heads, head_dim,
                             parts_for(max_context_len, partition_size));
}

extern "C" int32_t pa_decode_plan_capacity(int32_t num_seqs, int32_t max_context_len,
                                           int32_t block_size) {
  if (num_seqs <= 0) return 0;
  const int64_t per = block_size > 0 && max_context_len > 0
                          ? (static_cast<int64_t>(max_context_len) + block_size - 1) / block_size
                          : 1;
  const int64_t n = static_cast<int64_t>(num_seqs) * (per > 0 ? per : 1);
  return n > INT32_MAX ? INT32_MAX : static_cast<int32_t>(n);
}

extern "C" int pa_decode_plan(const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t q_dtype, int32_t partition_size, int32_t num_compute_units,
                              uint32_t* items, int32_t items_capacity, pkv_decode_plan* plan) {
  if (!plan) return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan: NULL plan");
  *plan = pkv_decode_plan{};
  if (num_seqs < 0 || num_seqs > 65535 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      block_size <= 0 || items_capacity < 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan: bad sizes");
  if (num_seqs > 0 && !context_lens) return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan: NULL lengths");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_UNSUPPORTED, "pa_decode_plan: num_q_heads %d not a multiple of %d",
                num_q_heads, num_kv_heads);
  if (q_dtype != PKV_F32 && q_dtype != PKV_F16)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan: q_dtype %d unknown", q_dtype);
  if (partition_size > 0 && partition_size % block_size != 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan: partition_size %d not a multiple of %d",
                partition_size, block_size);
  const KernelChoice kc = choose_kernel(q_dtype, num_q_heads / num_kv_heads);
  const int tiles = num_q_heads / kc.gt;
  // Per-thread scratch: a plan is made every decode step.
  static thread_local std::vector<int32_t> lens;
  static thread_local std::vector<uint64_t> keys;
  lens.resize(static_cast<size_t>(num_seqs));
  int32_t longest = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    lens[i] = context_lens[i] > 0 ? context_lens[i] : 0;
    longest = std::max(longest, lens[i]);
  }
  const int cus = num_compute_units > 0 ? num_compute_units : 256;
  const int32_t part =
      partition_size >= 0 ? partition_size : auto_partition(lens.data(), num_seqs, tiles, cus, block_size);
  const int64_t parts = parts_for(longest, part);
  if (parts > 65535) return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan: more than 65535 partitions");

  int64_t count = 0;
  for (int32_t i = 0; i < num_seqs; ++i) count += part > 0 && lens[i] > 0 ? (lens[i] + part - 1) / part : 1;
  plan->partition_size = part;
  plan->max_parts = static_cast<int32_t>(parts);
  plan->num_items = count > INT32_MAX ? INT32_MAX : static_cast<int32_t>(count);
  plan->waves_per_cu = residency_limit(kc.mfma, part, lens.data(), num_seqs);
  plan->workspace_bytes = workspace_bytes_for(num_seqs, num_q_heads, head_dim, parts);
  if (count > items_capacity)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan: %lld items do not fit in %d",
                static_cast<long long>(count), items_capacity);
  if (count > 0 && !items) return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan: NULL items");

  // Item order.  Requests by length, longest first (ties: lower index), as
  // ascending 64-bit keys (complemented length, index).  Full partitions (all
  // of one size) come first, request by request; then the requests' shorter
  // last pieces by size, largest first (ties: the request's rank above).
  keys.resize(static_cast<size_t>(num_seqs));
  for (int32_t i = 0; i < num_seqs; ++i)
    keys[i] = (static_cast<uint64_t>(UINT32_MAX - static_cast<uint32_t>(lens[i])) << 32) |
              static_cast<uint32_t>(i);
  std::sort(keys.begin(), keys.end());
  int64_t k = 0;
  if (part > 0) {
    for (int32_t r = 0; r < num_seqs; ++r) {
      const int32_t s = static_cast<int32_t>(keys[r] & 0xFFFFFFFFu);
      for (int32_t j = 0; j < lens[s] / part; ++j) items[k++] = PKV_ITEM(s, j);
    }
  }
  // Tail keys replace the request keys in place: (complemented tail size, rank),
  // with the request index recovered from the rank through a second array.
  static thread_local std::vector<int32_t> by_rank;
  by_rank.resize(static_cast<size_t>(num_seqs));
  int32_t ntails = 0;
  for (int32_t r = 0; r < num_seqs; ++r) {
    const int32_t s = static_cast<int32_t>(keys[r] & 0xFFFFFFFFu);
    by_rank[r] = s;
    const int32_t rest = part > 0 ? lens[s] % part : lens[s];
    if (rest > 0 || lens[s] == 0)
      keys[ntails++] = (static_cast<uint64_t>(UINT32_MAX - static_cast<uint32_t>(rest)) << 32) |
                       static_cast<uint32_t>(r);
  }
  std::sort(keys.begin(), keys.begin() + ntails);
  for (int32_t t = 0; t < ntails; ++t) {
    const int32_t s = by_rank[keys[t] & 0xFFFFFFFFu];
    items[k++] = PKV_ITEM(s, part > 0 ? lens[s] / part : 0);
  }
  if (k != count) return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan: internal count mismatch");
  return PKV_OK;
}


// ---------------------------------------------------------------- prefix groups
//
// Parallel samples of one prompt map their prompt blocks to the same physical
// blocks, and beams share every block up to where they diverged ("Only 20.4%
// of your KV cache held actual tokens" (blog.teqners.com), section "The part
// everyone forgets: pages enable sharing, not just packing").  Decode reads a
// request's whole context every step, so a shared block is read once per
// request that holds it.  Grouping such requests lets one wave read the block
// once for all of them.

namespace pkv_plan {
namespace {

int32_t leading_equal(const int32_t* a, int32_t na, const int32_t* b, int32_t nb) {
  const int32_t n = std::min(na, nb);
  int32_t j = 0;
  while (j < n && a[j] == b[j]) ++j;
  return j;
}

// Requests sorted by their full block ids (equal lists keep index order), so
// that those sharing the longest prefixes are neighbours; then runs of
// neighbours become groups of at most max_members, a member joining only if
// the group's saving ((members - 1) x shared blocks) does not shrink.
// shared_blocks[i]: leading blocks request i holds in common with its group.
void form_groups(const int32_t* const* blocks, const int32_t* nfull, int32_t n,
                 int32_t max_members, std::vector<int32_t>& groups,
                 std::vector<int32_t>& shared_blocks, int64_t& saved_blocks) {
  groups.clear();
  shared_blocks.assign(static_cast<size_t>(n), 0);
  saved_blocks = 0;
  if (max_members < 2) return;
  // Requests by first block (integer keys), then, inside each run of equal
  // first blocks, by the rest of their blocks; a request alone in its run
  // shares nothing and is dropped.
  static thread_local std::vector<uint64_t> keys;
  static thread_local std::vector<int32_t> order;
  keys.clear();
  order.clear();
  for (int32_t i = 0; i < n; ++i)
    if (nfull[i] >= 1)
      keys.push_back(static_cast<uint64_t>(static_cast<uint32_t>(blocks[i][0])) << 32 |
                     static_cast<uint32_t>(i));
  std::sort(keys.begin(), keys.end());
  for (size_t a = 0; a < keys.size();) {
    size_t b = a + 1;
    while (b < keys.size() && keys[b] >> 32 == keys[a] >> 32) ++b;
    if (b - a >= 2) {
      // Every member of the run holds its first `lcp` blocks in common: order
      // them by what follows.
      const size_t start = order.size();
      const int32_t head = static_cast<int32_t>(keys[a] & 0xFFFFFFFFu);
      int32_t lcp = nfull[head];
      for (size_t i = a; i < b; ++i) {
        const int32_t m = static_cast<int32_t>(keys[i] & 0xFFFFFFFFu);
        order.push_back(m);
        lcp = std::min(lcp, leading_equal(blocks[head], lcp, blocks[m], nfull[m]));
      }
      std::stable_sort(order.begin() + start, order.end(), [&](int32_t x, int32_t y) {
        return std::lexicographical_compare(blocks[x] + lcp, blocks[x] + nfull[x],
                                            blocks[y] + lcp, blocks[y] + nfull[y]);
      });
    }
    a = b;
  }
  size_t k = 0;
  while (k < order.size()) {
    const int32_t first = order[k];
    int32_t common = nfull[first];
    size_t end = k + 1;
    while (end < order.size() && static_cast<int32_t>(end - k) < max_members) {
      const int32_t next = order[end];
      const int32_t c =
          std::min(common, leading_equal(blocks[first], nfull[first], blocks[next], nfull[next]));
      const int64_t members = static_cast<int64_t>(end - k);
      if (c == 0 || members * c < (members - 1) * static_cast<int64_t>(common)) break;
      common = c;
      ++end;
    }
    const int32_t members = static_cast<int32_t>(end - k);
    if (members >= 2 && common >= 1) {
      groups.push_back(members);
      for (size_t i = k; i < end; ++i) {
        groups.push_back(order[i]);
        shared_blocks[order[i]] = common;
      }
      groups.resize(groups.size() + (PKV_GROUP_STRIDE - 1 - members), -1);
      saved_blocks += static_cast<int64_t>(members - 1) * common;
      k = end;
    } else {
      ++k;
    }
  }
}

}  // namespace

int plan_with_groups(const int32_t* const* blocks, const int32_t* nfull, const int32_t* lens,
                     int32_t n, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t q_dtype, int32_t partition_size,
                     int32_t num_compute_units, std::vector<uint32_t>& items,
                     pkv_decode_plan* plan, std::vector<int32_t>& groups,
                     std::vector<uint32_t>& group_items, std::vector<int32_t>& shared_lens) {
  groups.clear();
  group_items.clear();
  shared_lens.clear();
  int32_t longest = 0;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    longest = std::max(longest, lens[i]);
    total += std::max(0, lens[i]);
  }
  auto plan_items = [&](int32_t part) {
    items.resize(static_cast<size_t>(std::max(1, pa_decode_plan_capacity(n, longest, block_size))));
    const int rc = pa_decode_plan(lens, n, num_q_heads, num_kv_heads, head_dim, block_size,
                                  q_dtype, part, num_compute_units, items.data(),
                                  static_cast<int32_t>(items.size()), plan);
    items.resize(rc == PKV_OK ? static_cast<size_t>(plan->num_items) : 0);
    return rc;
  };
  // Shapes the group kernel serves; anything else (bad arguments included, which
  // pa_decode_plan reports) plans without groups.
  const int group = num_kv_heads > 0 && num_q_heads % num_kv_heads == 0 ? num_q_heads / num_kv_heads : 0;
  if (q_dtype != PKV_F16 || group < 1 || group > 8 || n < 2 || block_size <= 0 ||
      (head_dim != 64 && head_dim != 128) || n > 65535 ||
      (partition_size > 0 && partition_size % block_size != 0))
    return plan_items(partition_size);
  static thread_local std::vector<int32_t> shared_blocks;
  int64_t saved_blocks = 0;
  form_groups(blocks, nfull, n, 16 / group, groups, shared_blocks, saved_blocks);
  if (groups.empty() || static_cast<double>(saved_blocks) * block_size <
                            kGroupMinSavedFraction * static_cast<double>(total)) {
    groups.clear();
    return plan_items(partition_size);
  }
  // The partition size the plain plan would take, or, for a one-pass plan, the
  // groups' own.
  int32_t part = partition_size;
  if (part < 0) {
    static thread_local std::vector<int32_t> clamped;
    clamped.resize(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) clamped[i] = std::max(0, lens[i]);
    const KernelChoice kc = choose_kernel(q_dtype, group);
    part = auto_partition(clamped.data(), n, num_q_heads / kc.gt,
                          num_compute_units > 0 ? num_compute_units : 256, block_size);
  }
  if (part == 0) part = (kGroupPartitionTokens + block_size - 1) / block_size * block_size;
  if (int rc = plan_items(part)) {
    groups.clear();
    return rc;
  }
  // Group pieces: every whole partition of the shared prefix, then, when the
  // prefix ends inside a partition, that partition up to the prefix's end (its
  // members' own pieces for it start there; shared_lens tells the kernels).
  shared_lens.assign(static_cast<size_t>(n), 0);
  const int32_t ngroups = static_cast<int32_t>(groups.size() / PKV_GROUP_STRIDE);
  for (int32_t g = 0; g < ngroups; ++g) {
    const int32_t* row = groups.data() + static_cast<size_t>(g) * PKV_GROUP_STRIDE;
    const int32_t ls = shared_blocks[row[1]] * block_size;
    const int32_t whole = ls / part;
    const int32_t pieces = whole + (ls % part != 0 ? 1 : 0);
    for (int32_t j = 0; j < pieces; ++j) group_items.push_back(PKV_ITEM(g, j));
    if (ls % part != 0)
      for (int32_t i = 1; i <= row[0]; ++i) shared_lens[row[i]] = ls;
  }
  // Remaining pieces: a member's partitions past the shared prefix, and the
  // partition the prefix ends in when the member has tokens past it.
  size_t kept = 0;
  for (size_t i = 0; i < items.size(); ++i) {
    const uint32_t it = items[i];
    const int32_t s = static_cast<int32_t>(it >> 16);
    const int32_t p = static_cast<int32_t>(it & 0xFFFFu);
    const int32_t ls = shared_blocks[s] * block_size;
    const bool covered = static_cast<int64_t>(p + 1) * part <= ls ||
                         (static_cast<int64_t>(p) * part < ls && lens[s] <= ls);
    if (!covered) items[kept++] = it;
  }
  items.resize(kept);
  plan->num_items = static_cast<int32_t>(kept);
  // One launch for both kinds of piece when the remaining ones carry at least
  // half the group pieces' token reads (measured on MI355X: parallel sampling,
  // ratio 1.15, 13% faster in one launch; beams, ratio 0.35, 4% slower).
  int64_t group_tokens = 0, rest_tokens = 0;
  for (uint32_t it : group_items) {
    const int32_t* row = groups.data() + static_cast<size_t>(it >> 16) * PKV_GROUP_STRIDE;
    const int64_t lo = static_cast<int64_t>(it & 0xFFFFu) * part;
    const int64_t ls = shared_blocks[row[1]] * block_size;
    group_tokens += std::min<int64_t>(lo + part, ls) - lo;
  }
  for (uint32_t it : items) {
    const int32_t s_ = static_cast<int32_t>(it >> 16);
    int64_t lo = static_cast<int64_t>(it & 0xFFFFu) * part;
    const int64_t ls = shared_blocks[s_] * block_size;
    if (ls > lo && ls < lo + part) lo = ls;
    rest_tokens += std::min<int64_t>(lo + part, std::max(0, lens[s_])) - lo;
  }
  plan->fuse_groups = 2 * rest_tokens >= group_tokens ? 1 : 0;
  // Partials per request: one more slot for a member whose own piece of the
  // boundary partition is separate from the group's.
  plan->workspace_bytes = workspace_bytes_for(n, num_q_heads, head_dim, plan->max_parts + 1);
  return PKV_OK;
}

}  // namespace pkv_plan

extern "C" int pa_decode_plan_groups(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t q_dtype, int32_t partition_size,
                                     int32_t num_compute_units, uint32_t* items,
                                     int32_t items_capacity, pkv_decode_plan* plan,
                                     int32_t* groups, int32_t groups_capacity,
                                     int32_t* num_groups, uint32_t* group_items,
                                     int32_t* num_group_items, int32_t* shared_lens) {
  if (!plan || !num_groups || !num_group_items)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan_groups: NULL output");
  *num_groups = 0;
  *num_group_items = 0;
  if (num_seqs < 0 || num_seqs > 65535 || max_blocks_per_seq < 0 || block_size <= 0 ||
      groups_capacity < 0 || items_capacity < 0)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan_groups: bad sizes");
  if (num_seqs > 0 && (!context_lens || (!block_tables && max_blocks_per_seq > 0)))
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan_groups: NULL input");
  static thread_local std::vector<const int32_t*> rows;
  static thread_local std::vector<int32_t> nfull, lens;
  static thread_local std::vector<uint32_t> rest, gitems;
  static thread_local std::vector<int32_t> gdesc, shared;
  rows.resize(static_cast<size_t>(num_seqs));
  nfull.resize(static_cast<size_t>(num_seqs));
  lens.resize(static_cast<size_t>(num_seqs));
  for (int32_t i = 0; i < num_seqs; ++i) {
    lens[i] = std::max(0, context_lens[i]);
    rows[i] = block_tables + static_cast<int64_t>(i) * max_blocks_per_seq;
    nfull[i] = std::min(lens[i] / block_size, max_blocks_per_seq);
  }
  if (int rc = plan_with_groups(rows.data(), nfull.data(), lens.data(), num_seqs, num_q_heads,
                                num_kv_heads, head_dim, block_size, q_dtype, partition_size,
                                num_compute_units, rest, plan, gdesc, gitems, shared))
    return rc;
  const int32_t ng = static_cast<int32_t>(gdesc.size() / PKV_GROUP_STRIDE);
  if (static_cast<int64_t>(rest.size()) > items_capacity ||
      static_cast<int64_t>(gitems.size()) > items_capacity)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan_groups: %zu + %zu items do not fit in %d",
                rest.size(), gitems.size(), items_capacity);
  if (ng > groups_capacity)
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan_groups: %d groups do not fit in %d", ng,
                groups_capacity);
  if ((!rest.empty() && !items) || (!gitems.empty() && !group_items) ||
      (ng > 0 && (!groups || !shared_lens)))
    return fail(PKV_ERR_INVALID_ARG, "pa_decode_plan_groups: NULL output array");
  if (!rest.empty()) std::memcpy(items, rest.data(), sizeof(uint32_t) * rest.size());
  if (!gitems.empty()) std::memcpy(group_items, gitems.data(), sizeof(uint32_t) * gitems.size());
  if (ng > 0) {
    std::memcpy(groups, gdesc.data(), sizeof(int32_t) * gdesc.size());
    std::memcpy(shared_lens, shared.data(), sizeof(int32_t) * shared.size());
  }
  *num_groups = ng;
  *num_group_items = static_cast<int32_t>(gitems.size());
  return PKV_OK;
}
