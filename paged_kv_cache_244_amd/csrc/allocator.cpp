// Host block allocator: block tables, reference counts, demand allocation,
// fork, copy-on-write and free for a paged KV cache.
//
// "Only 20.4% of your KV cache held actual tokens" (blog.teqners.com), sections
// "The page table, relocated into attention" (logical blocks filled left to
// right, a per-request table to physical blocks, a new block only when the last
// one is full) and "The part everyone forgets: pages enable sharing, not just
// packing" (shared blocks with reference counts; a write into a shared, partly
// filled block takes a fresh block that receives a copy; freed blocks at zero
// references return to the pool).  "The KV cache is a systems problem"
// (rsw.lol), section "Shared prefixes need ownership rules": other readers keep
// their view.  Same notes, section "Eviction and reuse can move costs
// elsewhere": an evicted request's state may move to another memory tier; here
// a pool of blocks in host memory (the host tier) with its own free list.
//
// Plain host C++, no HIP.  Free list: a stack whose first pops follow the
// caller's initial order; freed blocks are pushed and so handed out next.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "decode_plan.h"
#include "errors.h"
#include "pagedkv.h"

struct kv_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  struct Parked {
    int32_t block;
    int64_t epoch;
  };
  // One tier of blocks: the device pool, or the host pool swapped requests use.
  struct Tier {
    std::vector<int32_t> free_stack;   // back() is handed out next
    std::vector<int32_t> refcount;     // per physical block
    std::vector<Parked> parked;        // freed with an epoch tag, in free order
    std::vector<int32_t> set_refs;     // scratch of a swap, all zero between calls
  };
  Tier dev;
  Tier host;                           // empty until kv_allocator_add_host_tier
  struct Seq {
    bool live = false;
    bool swapped = false;              // blocks name host-tier blocks
    int64_t length = 0;
    int32_t pending = 0;               // scratch of kv_decode_step_host, 0 between calls
    std::vector<int32_t> blocks;       // logical -> physical
  };
  std::vector<Seq> seqs;               // indexed by id; ids never reused
  int32_t swapped_seqs = 0;
  int64_t swapped_out_blocks = 0;      // copies device -> host, ever
  int64_t swapped_in_blocks = 0;       // copies host -> device, ever
};

namespace {

using pkv::fail;

int64_t blocks_for(int64_t tokens, int32_t B) { return (tokens + B - 1) / B; }

int check_seq(const kv_allocator* a, int32_t seq) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "allocator is NULL");
  if (seq < 0 || seq >= static_cast<int32_t>(a->seqs.size()) || !a->seqs[seq].live)
    return fail(PKV_ERR_BAD_SEQ, "sequence %d is unknown or freed", seq);
  return PKV_OK;
}

// Live and with its blocks on the device (not swapped out).
int check_resident(const kv_allocator* a, int32_t seq) {
  if (int rc = check_seq(a, seq)) return rc;
  if (a->seqs[seq].swapped)
    return fail(PKV_ERR_SWAPPED, "sequence %d is swapped out to the host tier", seq);
  return PKV_OK;
}

// Fills a tier's free stack so that the first pop is initial_order[0].
int init_tier(kv_allocator::Tier& t, int32_t n, const int32_t* initial_order) {
  t.refcount.assign(n, 0);
  t.set_refs.assign(n, 0);
  t.free_stack.resize(n);
  t.parked.clear();
  std::vector<char> seen(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = initial_order ? initial_order[i] : i;
    if (b < 0 || b >= n || seen[b])
      return fail(PKV_ERR_INVALID_ARG, "initial_order is not a permutation of 0..%d", n - 1);
    seen[b] = 1;
    t.free_stack[n - 1 - i] = b;   // initial_order[0] on top
  }
  return PKV_OK;
}

// What one append did, enough to undo it exactly (for all-or-nothing batches).
struct AppendRecord {
  int32_t seq;
  int64_t old_length;
  int32_t cow_src;     // -1 if no copy-on-write
  int32_t cow_dst;
  int32_t new_blocks;  // fresh blocks pushed onto the table (after a CoW dst)
};

int32_t pop_block(kv_allocator* a) {
  int32_t b = a->dev.free_stack.back();
  a->dev.free_stack.pop_back();
  a->dev.refcount[b] = 1;
  return b;
}

// Blocks an append of n tokens to `s` needs, copy-on-write included.
int64_t blocks_needed(const kv_allocator* a, const kv_allocator::Seq& s, int64_t n, bool* cow) {
  const int32_t B = a->block_size;
  *cow = n > 0 && (s.length % B) != 0 && a->dev.refcount[s.blocks.back()] > 1;
  int64_t fresh = blocks_for(s.length + n, B) - static_cast<int64_t>(s.blocks.size());
  return fresh + (*cow ? 1 : 0);
}

// Precondition: the pool has enough blocks.  Writes n slots; returns the record.
AppendRecord do_append(kv_allocator* a, int32_t seq, int64_t n, int64_t* slots_out) {
  kv_allocator::Seq& s = a->seqs[seq];
  const int32_t B = a->block_size;
  bool cow = false;
  blocks_needed(a, s, n, &cow);
  AppendRecord rec{seq, s.length, -1, -1, 0};
  if (cow) {
    int32_t src = s.blocks.back();
    int32_t dst = pop_block(a);
    a->dev.refcount[src] -= 1;
    s.blocks.back() = dst;
    rec.cow_src = src;
    rec.cow_dst = dst;
  }
  for (int64_t t = s.length; t < s.length + n; ++t) {
    if (t % B == 0) {
      s.blocks.push_back(pop_block(a));
      rec.new_blocks += 1;
    }
    slots_out[t - s.length] = static_cast<int64_t>(s.blocks[t / B]) * B + (t % B);
  }
  s.length += n;
  return rec;
}

// Exact inverse of do_append, so the free stack returns to its prior order.
void undo_append(kv_allocator* a, const AppendRecord& rec) {
  kv_allocator::Seq& s = a->seqs[rec.seq];
  for (int32_t i = 0; i < rec.new_blocks; ++i) {
    int32_t b = s.blocks.back();
    s.blocks.pop_back();
    a->dev.refcount[b] = 0;
    a->dev.free_stack.push_back(b);
  }
  if (rec.cow_src >= 0) {
    a->dev.refcount[rec.cow_dst] = 0;
    a->dev.free_stack.push_back(rec.cow_dst);
    a->dev.refcount[rec.cow_src] += 1;
    s.blocks.back() = rec.cow_src;
  }
  s.length = rec.old_length;
}

}  // namespace

extern "C" {

int kv_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_order,
                        kv_allocator** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_blocks (%d) and block_size (%d) must be positive",
                num_blocks, block_size);
  kv_allocator* a = new (std::nothrow) kv_allocator;
  if (!a) return fail(PKV_ERR_INVALID_ARG, "out of host memory");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  if (int rc = init_tier(a->dev, num_blocks, initial_order)) {
    delete a;
    return rc;
  }
  *out = a;
  return PKV_OK;
}

int kv_allocator_add_host_tier(kv_allocator* a, int32_t num_host_blocks,
                               const int32_t* initial_order) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "allocator is NULL");
  if (!a->host.refcount.empty()) return fail(PKV_ERR_INVALID_ARG, "the host tier exists already");
  if (num_host_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_host_blocks must be positive (got %d)", num_host_blocks);
  if (int rc = init_tier(a->host, num_host_blocks, initial_order)) {
    a->host = kv_allocator::Tier{};
    return rc;
  }
  return PKV_OK;
}

void kv_allocator_destroy(kv_allocator* a) { delete a; }

int kv_seq_create(kv_allocator* a, int32_t* seq_out) {
  if (!a || !seq_out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (a->seqs.size() >= static_cast<size_t>(INT32_MAX))
    return fail(PKV_ERR_INVALID_ARG, "sequence ids exhausted");
  a->seqs.emplace_back();
  a->seqs.back().live = true;
  *seq_out = static_cast<int32_t>(a->seqs.size() - 1);
  return PKV_OK;
}

int kv_seq_fork(kv_allocator* a, int32_t parent, int32_t* child_out) {
  if (int rc = check_resident(a, parent)) return rc;
  if (!child_out) return fail(PKV_ERR_INVALID_ARG, "child_out is NULL");
  int32_t child = 0;
  if (int rc = kv_seq_create(a, &child)) return rc;
  kv_allocator::Seq& c = a->seqs[child];
  const kv_allocator::Seq& p = a->seqs[parent];   // after emplace_back: no dangling ref
  c.blocks = p.blocks;
  c.length = p.length;
  for (int32_t b : c.blocks) a->dev.refcount[b] += 1;
  *child_out = child;
  return PKV_OK;
}

int kv_seq_append(kv_allocator* a, int32_t seq, int32_t n, int64_t* slots_out,
                  int32_t* cow_pair_out, int32_t* n_cow_out) {
  if (int rc = check_resident(a, seq)) return rc;
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0 (got %d)", n);
  if ((n > 0 && !slots_out) || !cow_pair_out || !n_cow_out)
    return fail(PKV_ERR_INVALID_ARG, "NULL output pointer");
  *n_cow_out = 0;
  if (n == 0) return PKV_OK;
  bool cow = false;
  int64_t need = blocks_needed(a, a->seqs[seq], n, &cow);
  if (need > static_cast<int64_t>(a->dev.free_stack.size()))
    return fail(PKV_ERR_OUT_OF_BLOCKS, "append of %d tokens needs %lld blocks, %zu free", n,
                static_cast<long long>(need), a->dev.free_stack.size());
  AppendRecord rec = do_append(a, seq, n, slots_out);
  if (rec.cow_src >= 0) {
    cow_pair_out[0] = rec.cow_src;
    cow_pair_out[1] = rec.cow_dst;
    *n_cow_out = 1;
  }
  return PKV_OK;
}

int kv_batch_append(kv_allocator* a, const int32_t* seqs, int32_t num_seqs, int64_t* slots_out,
                    int32_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!a || !n_cow_out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs must be >= 0");
  *n_cow_out = 0;
  if (num_seqs == 0) return PKV_OK;
  if (!seqs || !slots_out || !cow_pairs_out) return fail(PKV_ERR_INVALID_ARG, "NULL array");
  std::vector<AppendRecord> done;
  done.reserve(num_seqs);
  int status = PKV_OK;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t seq = seqs[i];
    if ((status = check_resident(a, seq))) break;
    bool cow = false;
    int64_t need = blocks_needed(a, a->seqs[seq], 1, &cow);
    if (need > static_cast<int64_t>(a->dev.free_stack.size())) {
      status = fail(PKV_ERR_OUT_OF_BLOCKS, "decode step for %d sequences ran out of blocks at #%d",
                    num_seqs, i);
      break;
    }
    done.push_back(do_append(a, seq, 1, slots_out + i));
  }
  if (status != PKV_OK) {
    for (auto it = done.rbegin(); it != done.rend(); ++it) undo_append(a, *it);
    return status;
  }
  int32_t n = 0;
  for (const AppendRecord& r : done) {
    if (r.cow_src >= 0) {
      cow_pairs_out[2 * n] = r.cow_src;
      cow_pairs_out[2 * n + 1] = r.cow_dst;
      ++n;
    }
  }
  *n_cow_out = n;
  return PKV_OK;
}

namespace {

// Drops the sequence's references in logical order; a block reaching zero goes
// to its tier's free list, or is parked with `epoch` when `deferred`.
int release_seq(kv_allocator* a, int32_t seq, bool deferred, int64_t epoch) {
  if (int rc = check_seq(a, seq)) return rc;
  kv_allocator::Seq& s = a->seqs[seq];
  kv_allocator::Tier& t = s.swapped ? a->host : a->dev;
  for (int32_t b : s.blocks) {
    if (--t.refcount[b] == 0) {
      if (deferred)
        t.parked.push_back({b, epoch});
      else
        t.free_stack.push_back(b);
    }
  }
  s.blocks.clear();
  s.blocks.shrink_to_fit();
  s.length = 0;
  s.live = false;
  if (s.swapped) --a->swapped_seqs;
  s.swapped = false;
  return PKV_OK;
}

int32_t retire_tier(kv_allocator::Tier& t, int64_t done) {
  int32_t released = 0;
  size_t keep = 0;
  for (size_t i = 0; i < t.parked.size(); ++i) {
    const kv_allocator::Parked p = t.parked[i];
    if (p.epoch <= done) {
      t.free_stack.push_back(p.block);
      ++released;
    } else {
      t.parked[keep++] = p;
    }
  }
  t.parked.resize(keep);
  return released;
}

// Moves every block the listed sequences reference from tier `from` to tier
// `to`: each distinct block (request order, then logical order) gets one fresh
// block of `to` whose count is the set's references; the old block loses those
// references and, at zero, is freed or parked.  Checks everything first; on
// any error nothing changes.
int swap_set(kv_allocator* a, const int32_t* seqs, int32_t n, bool to_host, int32_t deferred,
             int64_t epoch, int32_t* pairs_out, int32_t pairs_capacity, int32_t* num_pairs_out) {
  if (!a || !num_pairs_out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  *num_pairs_out = 0;
  if (n < 0 || pairs_capacity < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
  if (n > 0 && !seqs) return fail(PKV_ERR_INVALID_ARG, "NULL seqs");
  std::vector<int32_t> sorted(seqs, seqs + n);
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
    return fail(PKV_ERR_INVALID_ARG, "a sequence is listed twice");
  for (int32_t i = 0; i < n; ++i) {
    if (int rc = check_seq(a, seqs[i])) return rc;
    if (a->seqs[seqs[i]].swapped == to_host)
      return fail(PKV_ERR_SWAPPED, "sequence %d is %s", seqs[i],
                  to_host ? "swapped out already" : "not swapped out");
  }
  kv_allocator::Tier& from = to_host ? a->dev : a->host;
  kv_allocator::Tier& to = to_host ? a->host : a->dev;
  // Distinct blocks, first appearance first; set_refs counts the set's references.
  std::vector<int32_t> order;
  for (int32_t i = 0; i < n; ++i)
    for (int32_t b : a->seqs[seqs[i]].blocks)
      if (from.set_refs[b]++ == 0) order.push_back(b);
  const int32_t distinct = static_cast<int32_t>(order.size());
  int status = PKV_OK;
  if (distinct > 0 && !pairs_out)
    status = fail(PKV_ERR_INVALID_ARG, "NULL pairs_out");
  else if (distinct > pairs_capacity)
    status = fail(PKV_ERR_INVALID_ARG, "%d pairs needed, capacity %d", distinct, pairs_capacity);
  else if (distinct > static_cast<int32_t>(to.free_stack.size()))
    status = fail(PKV_ERR_OUT_OF_BLOCKS, "swap %s needs %d blocks, %zu free",
                  to_host ? "out" : "in", distinct, to.free_stack.size());
  if (status != PKV_OK) {
    for (int32_t b : order) from.set_refs[b] = 0;
    if (distinct > pairs_capacity) *num_pairs_out = distinct;
    return status;
  }
  // new_of: reuse set_refs as old block -> new block after taking the counts.
  for (int32_t j = 0; j < distinct; ++j) {
    const int32_t b = order[j];
    const int32_t refs = from.set_refs[b];
    const int32_t nb = to.free_stack.back();
    to.free_stack.pop_back();
    to.refcount[nb] = refs;
    from.refcount[b] -= refs;
    if (from.refcount[b] == 0) {
      if (deferred)
        from.parked.push_back({b, epoch});
      else
        from.free_stack.push_back(b);
    }
    from.set_refs[b] = nb;
    pairs_out[2 * j] = b;
    pairs_out[2 * j + 1] = nb;
  }
  for (int32_t i = 0; i < n; ++i) {
    kv_allocator::Seq& s = a->seqs[seqs[i]];
    for (int32_t& b : s.blocks) b = from.set_refs[b];
    s.swapped = to_host;
  }
  for (int32_t b : order) from.set_refs[b] = 0;
  a->swapped_seqs += to_host ? n : -n;
  (to_host ? a->swapped_out_blocks : a->swapped_in_blocks) += distinct;
  *num_pairs_out = distinct;
  return PKV_OK;
}

}  // namespace

int kv_seq_free(kv_allocator* a, int32_t seq) { return release_seq(a, seq, false, 0); }

int kv_seq_free_deferred(kv_allocator* a, int32_t seq, int64_t epoch) {
  return release_seq(a, seq, true, epoch);
}

int kv_allocator_retire(kv_allocator* a, int64_t done, int32_t* released_out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "allocator is NULL");
  const int32_t released = retire_tier(a->dev, done) + retire_tier(a->host, done);
  if (released_out) *released_out = released;
  return PKV_OK;
}

int kv_swap_out(kv_allocator* a, const int32_t* seqs, int32_t num_seqs, int32_t deferred,
                int64_t epoch, int32_t* pairs_out, int32_t pairs_capacity,
                int32_t* num_pairs_out) {
  return swap_set(a, seqs, num_seqs, true, deferred, epoch, pairs_out, pairs_capacity,
                  num_pairs_out);
}

int kv_swap_in(kv_allocator* a, const int32_t* seqs, int32_t num_seqs, int32_t deferred,
               int64_t epoch, int32_t* pairs_out, int32_t pairs_capacity,
               int32_t* num_pairs_out) {
  return swap_set(a, seqs, num_seqs, false, deferred, epoch, pairs_out, pairs_capacity,
                  num_pairs_out);
}

int kv_seq_is_swapped(const kv_allocator* a, int32_t seq, int32_t* swapped_out) {
  if (int rc = check_seq(a, seq)) return rc;
  if (!swapped_out) return fail(PKV_ERR_INVALID_ARG, "swapped_out is NULL");
  *swapped_out = a->seqs[seq].swapped ? 1 : 0;
  return PKV_OK;
}

int kv_seq_len(const kv_allocator* a, int32_t seq, int32_t* len_out) {
  if (int rc = check_seq(a, seq)) return rc;
  if (!len_out) return fail(PKV_ERR_INVALID_ARG, "len_out is NULL");
  if (a->seqs[seq].length > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "length overflows int32");
  *len_out = static_cast<int32_t>(a->seqs[seq].length);
  return PKV_OK;
}

int kv_seq_lens(const kv_allocator* a, const int32_t* seqs, int32_t n, int32_t* lens_out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "allocator is NULL");
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
  if (n > 0 && (!seqs || !lens_out)) return fail(PKV_ERR_INVALID_ARG, "NULL array");
  for (int32_t i = 0; i < n; ++i) {
    if (int rc = check_seq(a, seqs[i])) return rc;
    if (a->seqs[seqs[i]].length > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "length overflows int32");
  }
  for (int32_t i = 0; i < n; ++i) lens_out[i] = static_cast<int32_t>(a->seqs[seqs[i]].length);
  return PKV_OK;
}

int kv_export_block_tables(const kv_allocator* a, const int32_t* seqs, int32_t n,
                           int32_t max_blocks_per_seq, int32_t pad_value, int32_t* tables_out,
                           int32_t* lens_out) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "allocator is NULL");
  if (n < 0 || max_blocks_per_seq < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
  if (n > 0 && (!seqs || !tables_out || !lens_out)) return fail(PKV_ERR_INVALID_ARG, "NULL array");
  for (int32_t i = 0; i < n; ++i) {
    if (int rc = check_resident(a, seqs[i])) return rc;
    const kv_allocator::Seq& s = a->seqs[seqs[i]];
    if (static_cast<int64_t>(s.blocks.size()) > max_blocks_per_seq)
      return fail(PKV_ERR_INVALID_ARG, "sequence %d holds %zu blocks > max_blocks_per_seq %d",
                  seqs[i], s.blocks.size(), max_blocks_per_seq);
    if (s.length > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "length overflows int32");
  }
  for (int32_t i = 0; i < n; ++i) {
    const kv_allocator::Seq& s = a->seqs[seqs[i]];
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks_per_seq;
    size_t nb = s.blocks.size();
    for (size_t j = 0; j < nb; ++j) row[j] = s.blocks[j];
    for (int32_t j = static_cast<int32_t>(nb); j < max_blocks_per_seq; ++j) row[j] = pad_value;
    lens_out[i] = static_cast<int32_t>(s.length);
  }
  return PKV_OK;
}

int kv_decode_step_host(kv_allocator* a, const int32_t* seqs, int32_t num_seqs,
                        int32_t max_blocks_per_seq, int32_t pad_value, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t q_dtype,
                        int32_t partition_size, int32_t num_compute_units, int32_t flags,
                        void* buffer, uint64_t buffer_bytes, kv_step_layout* layout) {
  if (!a || !layout) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (flags & ~static_cast<int32_t>(PKV_STEP_GROUPS))
    return fail(PKV_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  *layout = kv_step_layout{};
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs %d outside [0, 65535]", num_seqs);
  if (num_seqs > 0 && !seqs) return fail(PKV_ERR_INVALID_ARG, "NULL seqs");
  const int32_t B = a->block_size;
  // Final lengths per entry (a sequence listed k times grows by k).
  for (int32_t i = 0; i < num_seqs; ++i)
    if (int rc = check_resident(a, seqs[i])) return rc;
  for (int32_t i = 0; i < num_seqs; ++i) a->seqs[seqs[i]].pending += 1;
  static thread_local std::vector<int32_t> lens;
  lens.resize(static_cast<size_t>(num_seqs));
  int64_t longest = 0, blocks_wanted = 0;
  bool too_long = false;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const kv_allocator::Seq& s = a->seqs[seqs[i]];
    const int64_t len = s.length + s.pending;
    too_long |= len > INT32_MAX;
    lens[i] = static_cast<int32_t>(len > INT32_MAX ? INT32_MAX : len);
    longest = std::max(longest, len);
    blocks_wanted = std::max(blocks_wanted, blocks_for(len, B));
  }
  for (int32_t i = 0; i < num_seqs; ++i) a->seqs[seqs[i]].pending = 0;
  if (too_long) return fail(PKV_ERR_INVALID_ARG, "length overflows int32");
  int32_t width = max_blocks_per_seq;
  if (width <= 0) width = static_cast<int32_t>(std::max<int64_t>(1, blocks_wanted));
  if (blocks_wanted > width)
    return fail(PKV_ERR_INVALID_ARG, "a sequence needs %lld blocks > max_blocks_per_seq %d",
                static_cast<long long>(blocks_wanted), width);
  // The plan, into scratch first: its size decides the layout.  Prefix groups
  // come from the blocks that are full before the append: the append leaves
  // them as they are (only a partly filled last block can be copied on write),
  // so they are what the tables hold after it.
  static thread_local std::vector<uint32_t> items, group_items;
  static thread_local std::vector<int32_t> groups, nfull, shared_lens;
  static thread_local std::vector<const int32_t*> rows;
  pkv_decode_plan plan{};
  rows.resize(static_cast<size_t>(num_seqs));
  nfull.resize(static_cast<size_t>(num_seqs));
  for (int32_t i = 0; i < num_seqs; ++i) {
    const kv_allocator::Seq& s = a->seqs[seqs[i]];
    rows[i] = s.blocks.data();
    nfull[i] = (flags & PKV_STEP_GROUPS) ? static_cast<int32_t>(s.length / B) : 0;
  }
  if (int rc = pkv_plan::plan_with_groups(rows.data(), nfull.data(), lens.data(), num_seqs,
                                          num_q_heads, num_kv_heads, head_dim, B, q_dtype,
                                          partition_size, num_compute_units, items, &plan, groups,
                                          group_items, shared_lens))
    return rc;
  auto up16 = [](uint64_t x) { return (x + 15) & ~static_cast<uint64_t>(15); };
  kv_step_layout L{};
  L.slots_offset = 0;
  L.pairs_offset = up16(L.slots_offset + 8ull * num_seqs);
  L.tables_offset = up16(L.pairs_offset + 8ull * num_seqs);
  L.lens_offset = up16(L.tables_offset + 4ull * num_seqs * static_cast<uint64_t>(width));
  L.items_offset = up16(L.lens_offset + 4ull * num_seqs);
  L.groups_offset = up16(L.items_offset + 4ull * static_cast<uint64_t>(plan.num_items));
  L.group_items_offset = up16(L.groups_offset + 4ull * groups.size());
  L.shared_lens_offset = up16(L.group_items_offset + 4ull * group_items.size());
  L.total_bytes = up16(L.shared_lens_offset + 4ull * shared_lens.size());
  L.num_groups = static_cast<int32_t>(groups.size() / PKV_GROUP_STRIDE);
  L.num_group_items = static_cast<int32_t>(group_items.size());
  L.max_blocks = width;
  L.max_context_len = static_cast<int32_t>(longest);
  L.plan = plan;
  if (!buffer || buffer_bytes < L.total_bytes) {
    layout->total_bytes = L.total_bytes;
    return fail(PKV_ERR_INVALID_ARG, "step buffer of %llu bytes needed (got %llu)",
                static_cast<unsigned long long>(L.total_bytes),
                static_cast<unsigned long long>(buffer ? buffer_bytes : 0));
  }
  char* base = static_cast<char*>(buffer);
  int32_t n_pairs = 0;
  if (int rc = kv_batch_append(a, seqs, num_seqs, reinterpret_cast<int64_t*>(base + L.slots_offset),
                               reinterpret_cast<int32_t*>(base + L.pairs_offset), &n_pairs))
    return rc;
  L.num_pairs = n_pairs;
  int32_t* tables = reinterpret_cast<int32_t*>(base + L.tables_offset);
  int32_t* lens_out = reinterpret_cast<int32_t*>(base + L.lens_offset);
  for (int32_t i = 0; i < num_seqs; ++i) {
    const kv_allocator::Seq& s = a->seqs[seqs[i]];
    int32_t* row = tables + static_cast<int64_t>(i) * width;
    const int32_t nb = static_cast<int32_t>(s.blocks.size());
    if (nb > 0) std::memcpy(row, s.blocks.data(), sizeof(int32_t) * nb);
    for (int32_t j = nb; j < width; ++j) row[j] = pad_value;
    lens_out[i] = static_cast<int32_t>(s.length);
  }
  if (plan.num_items > 0)
    std::memcpy(base + L.items_offset, items.data(), sizeof(uint32_t) * plan.num_items);
  if (!groups.empty()) std::memcpy(base + L.groups_offset, groups.data(), 4 * groups.size());
  if (!group_items.empty())
    std::memcpy(base + L.group_items_offset, group_items.data(), 4 * group_items.size());
  if (!shared_lens.empty())
    std::memcpy(base + L.shared_lens_offset, shared_lens.data(), 4 * shared_lens.size());
  *layout = L;
  return PKV_OK;
}

int kv_allocator_stats(const kv_allocator* a, kv_stats* out) {
  if (!a || !out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  kv_stats st{};
  st.num_blocks = a->num_blocks;
  st.free_blocks = static_cast<int32_t>(a->dev.free_stack.size());
  for (int32_t r : a->dev.refcount) {
    st.used_blocks += r > 0;
    st.shared_blocks += r > 1;
    st.sum_refcounts += r;
  }
  for (const kv_allocator::Seq& s : a->seqs)
    if (s.live) st.live_tokens += s.length;
  st.pending_blocks = static_cast<int32_t>(a->dev.parked.size());
  st.host_blocks = static_cast<int32_t>(a->host.refcount.size());
  st.host_free_blocks = static_cast<int32_t>(a->host.free_stack.size());
  for (int32_t r : a->host.refcount) st.host_used_blocks += r > 0;
  st.host_pending_blocks = static_cast<int32_t>(a->host.parked.size());
  st.swapped_seqs = a->swapped_seqs;
  st.swapped_out_blocks = a->swapped_out_blocks;
  st.swapped_in_blocks = a->swapped_in_blocks;
  *out = st;
  return PKV_OK;
}

}  // extern "C"
