"""Reference model of the paged block allocator (oracle; test infrastructure only).

Plain Python lists and dicts.  The rules, each from the pages:

* Fixed-size blocks of B token slots; a request fills its logical blocks left
  to right and a table maps each to a physical block (teqners explainer,
  section "The page table, relocated into attention").
* Demand allocation: a new physical block is taken only when every earlier
  block of the request is full (same section).
* Sharing: a forked request points at the same physical blocks; each block
  keeps a reference count (teqners explainer, section "The part everyone
  forgets: pages enable sharing, not just packing"; "800 kilobytes per token",
  section "The old answer, imported honestly").
* Copy-on-write: a request about to write into a shared, partly filled last
  block takes a fresh block, asks for one block's worth of data to be copied
  into it, and drops its reference to the shared one (same sections; rsw.lol,
  section "Shared prefixes need ownership rules": the other readers' view must
  be preserved).
* Freeing drops one reference per block; a block whose count reaches zero goes
  back to the pool (teqners explainer, sharing section).
* A block may be held back from reuse until device work still queued against
  it has finished (rsw.lol, section "Shared prefixes need ownership rules":
  storage must not be reassigned under a delayed device operation).
* Eviction may move a request's state to another memory tier instead of
  dropping it, at the price of the transfer (rsw.lol, section "Eviction and
  reuse can move costs elsewhere").  Here the other tier is a pool of blocks in
  host memory with the same block geometry; a request's state is its blocks.

Readings where the pages are silent:

* Free-list order: the caller gives the initial order; the first allocation
  returns ``initial_order[0]``, then ``[1]``...; a freed block is handed out
  next (last in, first out).  A request's blocks are released in logical order.
* Copy-on-write happens iff the append writes into a last block that is partly
  filled and has a count above one.  A full shared block is never written; the
  next token goes to a new block.  A request holding the last reference writes
  in place.  At most one copy per append.
* Running out of blocks changes nothing (the whole call fails).
* Request ids count up from 0 and are never reused.
* Deferred free: references drop at once, but a block reaching zero is parked
  with the caller's epoch; ``retire(done)`` returns every parked block with
  epoch <= done to the free list in the order they were freed.
* Swap moves a set of requests between the tiers together.  Each distinct
  block they reference (taken in request order, then logical order) is copied
  once into a fresh block of the other tier, so blocks shared inside the set
  stay shared; the new block's count is the number of the set's references,
  and the old block loses exactly those references (a block also held outside
  the set stays where it is for its other holders).  An old block left with no
  references is freed, or parked with an epoch as in a deferred free, since the
  queued copy still reads it.  All or nothing: too few free blocks in the
  target tier changes nothing.  A swapped-out request keeps its length and can
  be freed, but cannot grow, fork or be attended to until swapped back in.
  The host tier has its own free list with the same ordering rules.
"""

import copy


class OutOfBlocks(Exception):
    """The pool has fewer free blocks than the call needs; nothing changed."""


class BadSequence(Exception):
    """Unknown or already freed request id."""


class Swapped(Exception):
    """The request's blocks are in the host tier (or, for swap-in, are not)."""


class AllocatorModel:
    def __init__(self, num_blocks, block_size, initial_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if initial_order is None else [int(b) for b in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(reversed(order))      # top of stack = end of list
        self.refcount = [0] * num_blocks
        self.parked = []                        # (block, epoch) in free order
        self.tables = {}                        # seq id -> list of physical blocks
        self.lengths = {}                       # seq id -> tokens stored
        self.next_id = 0
        # host tier (empty until add_host_tier)
        self.host_blocks = 0
        self.host_free = []
        self.host_refcount = []
        self.host_parked = []
        self.swapped = set()                    # ids whose tables name host blocks
        self.swapped_out_blocks = 0             # blocks copied device -> host, ever
        self.swapped_in_blocks = 0              # blocks copied host -> device, ever

    def add_host_tier(self, num_host_blocks, initial_order=None):
        if self.host_blocks:
            raise ValueError("the host tier exists already")
        if num_host_blocks <= 0:
            raise ValueError("num_host_blocks must be positive")
        order = (list(range(num_host_blocks)) if initial_order is None
                 else [int(b) for b in initial_order])
        if sorted(order) != list(range(num_host_blocks)):
            raise ValueError("initial_order must be a permutation of 0..num_host_blocks-1")
        self.host_blocks = num_host_blocks
        self.host_free = list(reversed(order))
        self.host_refcount = [0] * num_host_blocks

    # -- requests ---------------------------------------------------------
    def _check(self, seq):
        if seq not in self.tables:
            raise BadSequence(seq)

    def _check_resident(self, seq):
        self._check(seq)
        if seq in self.swapped:
            raise Swapped(seq)

    def create(self):
        seq = self.next_id
        self.next_id += 1
        self.tables[seq] = []
        self.lengths[seq] = 0
        return seq

    def fork(self, parent):
        self._check_resident(parent)
        child = self.create()
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1
        return child

    def _pop(self):
        b = self.free.pop()
        self.refcount[b] = 1
        return b

    def append(self, seq, n):
        """Reserve slots for ``n`` more tokens.  Returns ``(slots, cow_pairs)``."""
        self._check_resident(seq)
        if n < 0:
            raise ValueError("n must be >= 0")
        if n == 0:
            return [], []
        B = self.block_size
        table, length = self.tables[seq], self.lengths[seq]
        cow = length % B != 0 and self.refcount[table[-1]] > 1
        held = len(table)
        wanted = (length + n + B - 1) // B
        need = (wanted - held) + (1 if cow else 0)
        if need > len(self.free):
            raise OutOfBlocks(need)
        pairs = []
        if cow:
            src = table[-1]
            dst = self._pop()
            self.refcount[src] -= 1
            table[-1] = dst
            pairs.append((src, dst))
        slots = []
        for t in range(length, length + n):
            if t % B == 0:
                table.append(self._pop())
            slots.append(table[t // B] * B + t % B)
        self.lengths[seq] = length + n
        return slots, pairs

    def append_batch(self, seqs):
        """One token for each listed request, in order; all or nothing."""
        saved = copy.deepcopy((self.free, self.refcount, self.tables, self.lengths))
        slots, pairs = [], []
        try:
            for seq in seqs:
                s, p = self.append(seq, 1)
                slots.extend(s)
                pairs.extend(p)
        except (OutOfBlocks, BadSequence, Swapped):
            self.free, self.refcount, self.tables, self.lengths = saved
            raise
        return slots, pairs

    def _tier(self, seq):
        """(reference counts, free list, parked list) of the tier holding ``seq``."""
        if seq in self.swapped:
            return self.host_refcount, self.host_free, self.host_parked
        return self.refcount, self.free, self.parked

    def free_seq(self, seq):
        self._check(seq)
        refcount, free, _ = self._tier(seq)
        for b in self.tables[seq]:
            refcount[b] -= 1
            if refcount[b] == 0:
                free.append(b)
        del self.tables[seq]
        del self.lengths[seq]
        self.swapped.discard(seq)

    def free_seq_deferred(self, seq, epoch):
        self._check(seq)
        refcount, _, parked = self._tier(seq)
        for b in self.tables[seq]:
            refcount[b] -= 1
            if refcount[b] == 0:
                parked.append((b, int(epoch)))
        del self.tables[seq]
        del self.lengths[seq]
        self.swapped.discard(seq)

    def retire(self, done):
        """Free every parked block (both tiers) with epoch <= done; how many."""
        released = [b for b, e in self.parked if e <= done]
        self.parked = [(b, e) for b, e in self.parked if e > done]
        self.free.extend(released)
        host_released = [b for b, e in self.host_parked if e <= done]
        self.host_parked = [(b, e) for b, e in self.host_parked if e > done]
        self.host_free.extend(host_released)
        return len(released) + len(host_released)

    # -- the host tier ------------------------------------------------------
    def _distinct_blocks(self, seqs):
        """The blocks the set references, first appearance first, with the set's
        reference count of each."""
        order, refs = [], {}
        for seq in seqs:
            for b in self.tables[seq]:
                if b not in refs:
                    order.append(b)
                    refs[b] = 0
                refs[b] += 1
        return order, refs

    def _check_set(self, seqs, want_swapped):
        if len(set(seqs)) != len(seqs):
            raise ValueError("a request is listed twice")
        for seq in seqs:
            self._check(seq)
            if (seq in self.swapped) != want_swapped:
                raise Swapped(seq)

    def swap_out(self, seqs, deferred=False, epoch=0):
        """Move the requests' blocks to the host tier.  Returns the copies to make,
        ``[(device block, host block), ...]``."""
        seqs = [int(s) for s in seqs]
        self._check_set(seqs, want_swapped=False)
        order, refs = self._distinct_blocks(seqs)
        if len(order) > len(self.host_free):
            raise OutOfBlocks(len(order))
        new_of, pairs = {}, []
        for b in order:
            h = self.host_free.pop()
            self.host_refcount[h] = refs[b]
            new_of[b] = h
            pairs.append((b, h))
            self.refcount[b] -= refs[b]
            if self.refcount[b] == 0:
                if deferred:
                    self.parked.append((b, int(epoch)))
                else:
                    self.free.append(b)
        for seq in seqs:
            self.tables[seq] = [new_of[b] for b in self.tables[seq]]
            self.swapped.add(seq)
        self.swapped_out_blocks += len(pairs)
        return pairs

    def swap_in(self, seqs, deferred=False, epoch=0):
        """Move swapped-out requests' blocks back to the device pool.  Returns the
        copies to make, ``[(host block, device block), ...]``."""
        seqs = [int(s) for s in seqs]
        self._check_set(seqs, want_swapped=True)
        order, refs = self._distinct_blocks(seqs)
        if len(order) > len(self.free):
            raise OutOfBlocks(len(order))
        new_of, pairs = {}, []
        for h in order:
            b = self.free.pop()
            self.refcount[b] = refs[h]
            new_of[h] = b
            pairs.append((h, b))
            self.host_refcount[h] -= refs[h]
            if self.host_refcount[h] == 0:
                if deferred:
                    self.host_parked.append((h, int(epoch)))
                else:
                    self.host_free.append(h)
        for seq in seqs:
            self.tables[seq] = [new_of[h] for h in self.tables[seq]]
            self.swapped.discard(seq)
        self.swapped_in_blocks += len(pairs)
        return pairs

    def is_swapped(self, seq):
        self._check(seq)
        return seq in self.swapped

    # -- views ------------------------------------------------------------
    def length(self, seq):
        self._check(seq)
        return self.lengths[seq]

    def table(self, seq):
        self._check(seq)
        return list(self.tables[seq])

    def export(self, seqs, max_blocks, pad_value):
        """Block tables ``[n][max_blocks]`` padded with ``pad_value``, and lengths."""
        rows, lens = [], []
        for seq in seqs:
            self._check_resident(seq)
            t = self.tables[seq]
            if len(t) > max_blocks:
                raise ValueError("sequence holds more blocks than max_blocks")
            rows.append(t + [pad_value] * (max_blocks - len(t)))
            lens.append(self.lengths[seq])
        return rows, lens

    def stats(self):
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": sum(1 for r in self.refcount if r > 0),
            "shared_blocks": sum(1 for r in self.refcount if r > 1),
            "live_tokens": sum(self.lengths.values()),
            "sum_refcounts": sum(self.refcount),
            "pending_blocks": len(self.parked),
            "host_blocks": self.host_blocks,
            "host_free_blocks": len(self.host_free),
            "host_used_blocks": sum(1 for r in self.host_refcount if r > 0),
            "host_pending_blocks": len(self.host_parked),
            "swapped_seqs": len(self.swapped),
            "swapped_out_blocks": self.swapped_out_blocks,
            "swapped_in_blocks": self.swapped_in_blocks,
        }
