"""The allocator model's host tier (swap out / swap in) against facts outside it.

"The KV cache is a systems problem" (rsw.lol), section "Eviction and reuse can
move costs elsewhere": evicted state may be moved to another memory tier
instead of being recomputed.  Moving it must not change it, and the move costs
transfer: each distinct block once.

Pins (none re-derives the model's own code):
* ground truth: every request's token list, kept by the test alone (a fork
  copies its parent's list, an append extends it).  After every operation of
  random histories the tokens read back through each request's table, in the
  tier that holds it, equal that list;
* queued copies: with deferred swaps the copies run late (another stream), while
  the host goes on appending and writing.  The tokens still read back right
  only if storage still read by a queued copy was not handed out;
* closed forms of sharing: n samples forked from one prompt and swapped
  together occupy ceil(P/B) host blocks (the prompt's), not n times as many;
  one sample swapped alone copies its blocks and the rest keep theirs;
* structural invariants of both tiers (every block free, parked or referenced
  exactly by the tables that hold it); all-or-nothing on exhaustion;
* copy-on-write after a round trip: a partly filled shared last block is still
  shared, so the next append copies it.
The last test runs these pins on planted mistakes and requires each caught.
"""

import copy

import numpy as np
import pytest

from oracle import cache as oc
from oracle import closed_forms as cf
from oracle.alloc_model import AllocatorModel, BadSequence, OutOfBlocks, Swapped

HKV, D = 2, 4


def check_invariants(m):
    dev_counts = [0] * m.num_blocks
    host_counts = [0] * m.host_blocks
    for seq, table in m.tables.items():
        assert len(table) == cf.blocks_for_tokens(m.lengths[seq], m.block_size)
        counts = host_counts if seq in m.swapped else dev_counts
        for b in table:
            counts[b] += 1
    assert dev_counts == m.refcount, "device count = tables holding the block"
    assert host_counts == m.host_refcount, "host count = tables holding the block"
    for n, refs, free, parked in ((m.num_blocks, m.refcount, m.free, m.parked),
                                  (m.host_blocks, m.host_refcount, m.host_free, m.host_parked)):
        idle = free + [b for b, _ in parked]
        assert len(set(idle)) == len(idle), "free and parked are disjoint, no repeats"
        assert all(refs[b] == 0 for b in idle), "an idle block has no holder"
        assert sum(1 for r in refs if r > 0) + len(idle) == n, "no block is lost"


class World:
    """The model plus device and host pools with real bytes, a ground-truth token
    list per request, and a queue of copies that run when their epoch completes.

    Writes run at once, as if on a stream of their own that does not wait for the
    copies.  A caller still orders its own work: before it writes a request whose
    copy is queued it waits for that copy, and an immediate (non-deferred) free or
    swap first waits for everything queued.  What deferral must cover is the rest:
    storage released while a queued copy still reads it, taken by someone else.
    """

    def __init__(self, model, nb, nh, B, rng, host_order=None):
        self.m = model
        self.m.add_host_tier(nh, host_order)
        self.B = B
        self.rng = rng
        self.dev = (np.full((nb, HKV, B, D), np.nan, np.float16),
                    np.full((nb, HKV, B, D), np.nan, np.float16))
        self.host = (np.full((nh, HKV, B, D), np.nan, np.float16),
                     np.full((nh, HKV, B, D), np.nan, np.float16))
        self.truth = {}
        self.queued = []          # (epoch, src pools, dst pools, pairs)
        self.pending = {}         # request -> epoch of its last queued copy
        self.epoch = 0
        self.counter = 0

    def _tokens(self, n):
        # distinct, exactly representable values so that any misplaced copy shows
        vals = np.arange(self.counter, self.counter + n * HKV * D, dtype=np.float64) % 2048
        self.counter += n * HKV * D
        return vals.astype(np.float16).reshape(n, HKV, D)

    def create(self):
        s = self.m.create()
        self.truth[s] = []
        return s

    def _wait_for(self, s):
        if s in self.pending:
            self.complete(self.pending[s])

    def fork(self, s):
        self._wait_for(s)
        c = self.m.fork(s)
        self.truth[c] = list(self.truth[s])
        return c

    def append(self, s, n):
        self._wait_for(s)
        slots, pairs = self.m.append(s, n)
        oc.copy_blocks([self.dev], pairs)
        tok = self._tokens(n)
        oc.write_slots(*self.dev, tok, tok + 1, slots, self.B)
        self.truth[s].extend(tok)

    def append_batch(self, seqs):
        for s in seqs:
            self._wait_for(s)
        slots, pairs = self.m.append_batch(seqs)
        oc.copy_blocks([self.dev], pairs)
        tok = self._tokens(len(seqs))
        oc.write_slots(*self.dev, tok, tok + 1, slots, self.B)
        for s, t in zip(seqs, tok):
            self.truth[s].append(t)
        return pairs

    def free(self, s, deferred=False):
        if deferred:
            self.epoch += 1
            self.m.free_seq_deferred(s, self.epoch)
        else:
            self.complete(self.epoch)
            self.m.free_seq(s)
        del self.truth[s]
        self.pending.pop(s, None)

    def swap_out(self, seqs, deferred=False):
        return self._swap(self.m.swap_out, seqs, self.dev, self.host, deferred)

    def swap_in(self, seqs, deferred=False):
        return self._swap(self.m.swap_in, seqs, self.host, self.dev, deferred)

    def _swap(self, move, seqs, src, dst, deferred):
        if not deferred:
            self.complete(self.epoch)
        epoch = self.epoch + 1 if deferred else self.epoch
        pairs = move(seqs, deferred, epoch)
        if deferred:
            self.epoch = epoch
            self.queued.append((epoch, src, dst, list(pairs)))
            for s in seqs:
                self.pending[s] = epoch
        else:
            oc.copy_blocks_between([src], [dst], pairs)
        return pairs

    def complete(self, done):
        """The device finishes every queued copy up to epoch ``done``; then retire."""
        keep = []
        for e, src, dst, pairs in self.queued:
            if e <= done:
                oc.copy_blocks_between([src], [dst], pairs)
            else:
                keep.append((e, src, dst, pairs))
        self.queued = keep
        self.pending = {s: e for s, e in self.pending.items() if e > done}
        self.m.retire(done)

    def check_views(self):
        if self.queued:
            return                 # a queued copy has not landed yet
        for s, toks in self.truth.items():
            pools = self.host if s in self.m.swapped else self.dev
            L = len(toks)
            assert self.m.lengths[s] == L
            if L == 0:
                continue
            want = np.array(toks)
            k = oc.gather_logical(pools[0], self.m.tables[s], L, self.B)
            v = oc.gather_logical(pools[1], self.m.tables[s], L, self.B)
            assert np.array_equal(k, want), f"request {s}: keys changed"
            assert np.array_equal(v, want + 1), f"request {s}: values changed"


def _random_history(make_model, seed, steps=200, nb=20, nh=16, B=4, deferred_p=0.0):
    rng = np.random.default_rng(seed)
    w = World(make_model(nb, B, rng.permutation(nb)), nb, nh, B, rng, rng.permutation(nh))
    live = []
    for _ in range(steps):
        op = int(rng.integers(9))
        try:
            if op == 0 or not live:
                live.append(w.create())
            elif op == 1:
                live.append(w.fork(live[rng.integers(len(live))]))
            elif op in (2, 3):
                w.append(live[rng.integers(len(live))], int(rng.integers(1, 2 * B + 1)))
            elif op == 4:
                w.free(live.pop(rng.integers(len(live))), deferred=rng.random() < deferred_p)
            elif op in (5, 6):
                want_out = op == 5
                pool = [s for s in live if (s in w.m.swapped) != want_out]
                if pool:
                    k = int(rng.integers(1, len(pool) + 1))
                    pick = [pool[i] for i in rng.choice(len(pool), size=k, replace=False)]
                    d = rng.random() < deferred_p
                    (w.swap_out if want_out else w.swap_in)(pick, deferred=d)
            elif op == 7:
                w.complete(int(rng.integers(0, w.epoch + 1)))
            else:
                w.complete(w.epoch)
        except (OutOfBlocks, Swapped):
            pass
        check_invariants(w.m)
        w.check_views()
    w.complete(w.epoch)
    w.check_views()
    return w, live


# -- pins (each takes a model class) -------------------------------------------

def pin_round_trips_preserve_tokens(make_model):
    for seed in range(12):
        _random_history(make_model, seed)


def pin_late_copies_still_preserve_tokens(make_model):
    for seed in range(12):
        _random_history(make_model, 100 + seed, deferred_p=0.7)


def pin_deferred_swap_out_then_other_writes(make_model):
    """Swap a request out with its copy still queued, then let another request take
    blocks and write at once: the queued copy must still read the old tokens."""
    rng = np.random.default_rng(3)
    w = World(make_model(6, 4, range(6)), 6, 6, 4, rng)
    a = w.create()
    w.append(a, 12)                             # 3 blocks
    w.swap_out([a], deferred=True)
    b = w.create()
    try:
        w.append(b, 12)                         # wants 3 blocks; only 3 are free
    except OutOfBlocks:
        raise AssertionError("a correct pool still has 3 free blocks") from None
    w.complete(w.epoch)
    w.check_views()
    check_invariants(w.m)


def pin_sampling_group_shares_host_blocks(make_model):
    B, P, n = 16, 100, 8
    rng = np.random.default_rng(1)
    w = World(make_model(64, B, None), 64, 64, B, rng)
    p = w.create()
    w.append(p, P)
    samples = [w.fork(p) for _ in range(n)]
    w.free(p)
    nb = cf.blocks_for_tokens(P, B)
    pairs = w.swap_out(samples)
    st = w.m.stats()
    assert len(pairs) == nb, "each distinct block is copied once"
    assert st["host_used_blocks"] == nb and st["used_blocks"] == 0
    assert st["free_blocks"] == 64
    pairs = w.swap_in(samples)
    assert len(pairs) == nb and w.m.stats()["used_blocks"] == nb
    assert w.m.stats()["host_used_blocks"] == 0
    # Still shared after the round trip: the first new token copies the partly
    # filled last block (P % B != 0) for all but the last holder.
    cow = w.append_batch(samples)
    assert len(cow) == n - 1
    check_invariants(w.m)
    w.check_views()


def pin_one_sample_swapped_alone(make_model):
    B, P = 8, 20
    rng = np.random.default_rng(2)
    w = World(make_model(32, B, None), 32, 32, B, rng)
    p = w.create()
    w.append(p, P)
    c = w.fork(p)
    nb = cf.blocks_for_tokens(P, B)
    pairs = w.swap_out([c])
    assert len(pairs) == nb and w.m.stats()["used_blocks"] == nb
    assert all(w.m.refcount[b] == 1 for b in w.m.tables[p])
    w.append(p, 1)                              # p now writes in place: no copy
    pairs = w.swap_in([c])
    assert len(pairs) == nb
    assert w.m.stats()["used_blocks"] == 2 * nb
    check_invariants(w.m)
    w.check_views()


def pin_swap_is_all_or_nothing(make_model):
    rng = np.random.default_rng(4)
    w = World(make_model(8, 2, None), 8, 3, 2, rng)
    a, b = w.create(), w.create()
    w.append(a, 4)                              # 2 blocks
    w.append(b, 4)                              # 2 blocks
    snap = copy.deepcopy(w.m.__dict__)
    with pytest.raises(OutOfBlocks):
        w.swap_out([a, b])                      # 4 blocks > 3 on the host
    assert w.m.__dict__ == snap
    w.swap_out([a])
    c = w.create()
    w.append(c, 12)                             # 6 blocks: the device is full
    snap = copy.deepcopy(w.m.__dict__)
    with pytest.raises(OutOfBlocks):
        w.swap_in([a])
    assert w.m.__dict__ == snap
    check_invariants(w.m)


def pin_swapped_request_rules(make_model):
    rng = np.random.default_rng(5)
    w = World(make_model(8, 2, None), 8, 8, 2, rng)
    a = w.create()
    w.append(a, 3)
    w.swap_out([a])
    for f in (lambda: w.m.append(a, 1), lambda: w.m.fork(a), lambda: w.m.export([a], 4, -1),
              lambda: w.m.append_batch([a]), lambda: w.m.swap_out([a])):
        with pytest.raises(Swapped):
            f()
    b = w.create()
    with pytest.raises(Swapped):
        w.m.swap_in([b])
    with pytest.raises(ValueError):
        w.m.swap_out([b, b])
    assert w.m.length(a) == 3 and w.m.stats()["swapped_seqs"] == 1
    w.free(a)
    st = w.m.stats()
    assert st["host_free_blocks"] == 8 and st["swapped_seqs"] == 0
    with pytest.raises(BadSequence):
        w.m.swap_in([a])
    check_invariants(w.m)


PINS = [pin_round_trips_preserve_tokens, pin_late_copies_still_preserve_tokens,
        pin_deferred_swap_out_then_other_writes, pin_sampling_group_shares_host_blocks,
        pin_one_sample_swapped_alone, pin_swap_is_all_or_nothing, pin_swapped_request_rules]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_model_passes_pin(pin):
    pin(AllocatorModel)


def test_swap_counters_and_exhaustive_short_histories():
    """Every sequence of up to 4 ops from a small alphabet (tiny pools), invariants
    and views after each; the counters add up the copies."""
    import itertools

    alphabet = ["create", "fork0", "app0_3", "applast_2", "out0", "outall", "in0", "inall",
                "free0"]
    for n in range(1, 5):
        for ops in itertools.product(alphabet, repeat=n):
            w = World(AllocatorModel(4, 2), 4, 3, 2, np.random.default_rng(0))
            live, copies_out, copies_in = [], 0, 0
            for op in ops:
                try:
                    if op == "create":
                        live.append(w.create())
                    elif not live:
                        continue
                    elif op == "fork0":
                        live.append(w.fork(live[0]))
                    elif op.startswith("app"):
                        w.append(live[0] if op.startswith("app0") else live[-1], int(op[-1]))
                    elif op.startswith("out"):
                        pick = [s for s in (live[:1] if op == "out0" else live)
                                if s not in w.m.swapped]
                        copies_out += len(w.swap_out(pick))
                    elif op.startswith("in"):
                        pick = [s for s in (live[:1] if op == "in0" else live) if s in w.m.swapped]
                        copies_in += len(w.swap_in(pick))
                    elif op == "free0":
                        w.free(live.pop(0))
                except (OutOfBlocks, Swapped):
                    pass
                check_invariants(w.m)
                w.check_views()
            st = w.m.stats()
            assert (st["swapped_out_blocks"], st["swapped_in_blocks"]) == (copies_out, copies_in)


# -- planted mistakes ------------------------------------------------------------

class _CopyPerReference(AllocatorModel):
    """Copies a shared block once per request instead of once."""

    def _distinct_blocks(self, seqs):
        order, refs = [], {}
        for seq in seqs:
            for b in self.tables[seq]:
                order.append(b)
                refs[b] = 1
        return order, refs

    def swap_out(self, seqs, deferred=False, epoch=0):
        seqs = [int(s) for s in seqs]
        self._check_set(seqs, want_swapped=False)
        if sum(len(self.tables[s]) for s in seqs) > len(self.host_free):
            raise OutOfBlocks()
        pairs = []
        for seq in seqs:
            new = []
            for b in self.tables[seq]:
                h = self.host_free.pop()
                self.host_refcount[h] = 1
                pairs.append((b, h))
                new.append(h)
                self.refcount[b] -= 1
                if self.refcount[b] == 0:
                    if deferred:
                        self.parked.append((b, int(epoch)))
                    else:
                        self.free.append(b)
            self.tables[seq] = new
            self.swapped.add(seq)
        self.swapped_out_blocks += len(pairs)
        return pairs


class _KeepsDeviceReferences(AllocatorModel):
    def swap_out(self, seqs, deferred=False, epoch=0):
        before = list(self.refcount)
        pairs = super().swap_out(seqs, deferred, epoch)
        for b, _ in pairs:                     # forgets to drop the set's references
            if b in self.free:
                self.free.remove(b)
            self.parked = [(x, e) for x, e in self.parked if x != b]
            self.refcount[b] = before[b]
        return pairs


class _FreesAtOnce(AllocatorModel):
    """Ignores ``deferred``: the device block goes back while the copy is queued."""

    def swap_out(self, seqs, deferred=False, epoch=0):
        return super().swap_out(seqs, False, epoch)


class _PairsReversed(AllocatorModel):
    def swap_in(self, seqs, deferred=False, epoch=0):
        return [(b, h) for h, b in super().swap_in(seqs, deferred, epoch)]


class _SecondHolderNotRemapped(AllocatorModel):
    """Remaps only the first request of the set to the copies."""

    def swap_in(self, seqs, deferred=False, epoch=0):
        seqs = [int(s) for s in seqs]
        old = {s: list(self.tables[s]) for s in seqs}
        pairs = super().swap_in(seqs, deferred, epoch)
        for s in seqs[1:]:
            self.tables[s] = old[s]
        return pairs


class _HostBlockNeverFreed(AllocatorModel):
    def swap_in(self, seqs, deferred=False, epoch=0):
        pairs = super().swap_in(seqs, deferred, epoch)
        for h, _ in pairs:
            if h in self.host_free:
                self.host_free.remove(h)
        return pairs


MUTANTS = {
    "copy_per_reference": _CopyPerReference,
    "keeps_device_references": _KeepsDeviceReferences,
    "frees_at_once_when_deferred": _FreesAtOnce,
    "swap_in_pairs_reversed": _PairsReversed,
    "second_holder_not_remapped": _SecondHolderNotRemapped,
    "host_block_never_freed": _HostBlockNeverFreed,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_swap_mutant_is_caught(name):
    caught = None
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(MUTANTS[name])
        except (AssertionError, IndexError, KeyError, ValueError, OutOfBlocks, Swapped):
            caught = pin.__name__
            break
    assert caught is not None, f"no pin catches {name}"
