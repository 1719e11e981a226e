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
"""

import copy


class OutOfBlocks(Exception):
    """The pool has fewer free blocks than the call needs; nothing changed."""


class BadSequence(Exception):
    """Unknown or already freed request id."""


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

    # -- requests ---------------------------------------------------------
    def _check(self, seq):
        if seq not in self.tables:
            raise BadSequence(seq)

    def create(self):
        seq = self.next_id
        self.next_id += 1
        self.tables[seq] = []
        self.lengths[seq] = 0
        return seq

    def fork(self, parent):
        self._check(parent)
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
        self._check(seq)
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
        except (OutOfBlocks, BadSequence):
            self.free, self.refcount, self.tables, self.lengths = saved
            raise
        return slots, pairs

    def free_seq(self, seq):
        self._check(seq)
        for b in self.tables[seq]:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.tables[seq]
        del self.lengths[seq]

    def free_seq_deferred(self, seq, epoch):
        self._check(seq)
        for b in self.tables[seq]:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.parked.append((b, int(epoch)))
        del self.tables[seq]
        del self.lengths[seq]

    def retire(self, done):
        released = [b for b, e in self.parked if e <= done]
        self.parked = [(b, e) for b, e in self.parked if e > done]
        self.free.extend(released)
        return len(released)

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
            self._check(seq)
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
        }
