"""The allocator model against the pages' rules, closed forms and invariants.

Pins (none re-derives the model's own code):
* block counts follow ceil(L/B) (the closed form pinned to the pages' 33-token
  example) and grow exactly when a block fills (demand allocation);
* a write through the slots followed by a gather through the table returns the
  tokens in logical order (write/gather are pinned by a library reshape);
* fork shares every block; copy-on-write in parallel sampling copies 7 of 8
  samples' last prompt block and leaves the other readers' view unchanged;
* structural invariants after every step of random and exhaustive op sequences;
* reclamation after everything is freed; all-or-nothing on exhaustion; LIFO reuse.
"""

import copy
import itertools

import numpy as np
import pytest

from oracle import cache as oc
from oracle import closed_forms as cf
from oracle.alloc_model import AllocatorModel, BadSequence, OutOfBlocks


def check_invariants(m: AllocatorModel):
    counts = [0] * m.num_blocks
    for seq, table in m.tables.items():
        assert len(table) == cf.blocks_for_tokens(m.lengths[seq], m.block_size)
        assert len(set(table)) == len(table), "a request never holds a block twice"
        for b in table:
            counts[b] += 1
    assert counts == m.refcount, "refcount = number of tables holding the block"
    parked = [b for b, _ in m.parked]
    assert len(set(m.free + parked)) == len(m.free) + len(parked), "free and parked are disjoint"
    for b in m.free + parked:
        assert m.refcount[b] == 0, "a free or parked block is referenced by nobody"
    used = sum(1 for r in m.refcount if r > 0)
    assert used + len(m.free) + len(parked) == m.num_blocks, \
        "no block is lost (no external fragmentation)"


def test_demand_allocation_and_block_count():
    m = AllocatorModel(64, 16)
    s = m.create()
    for t in range(100):
        before = len(m.table(s))
        slots, pairs = m.append(s, 1)
        assert pairs == []
        grew = len(m.table(s)) - before
        assert grew == (1 if t % 16 == 0 else 0), "new block only when the last is full"
    assert len(m.table(s)) == cf.blocks_for_tokens(100, 16) == 7
    check_invariants(m)


def test_33_tokens_three_blocks():
    m = AllocatorModel(8, 16)
    s = m.create()
    m.append(s, 33)
    assert len(m.table(s)) == 3
    assert 3 * 16 - m.length(s) == 15


def test_initial_order_and_lifo():
    order = [5, 2, 7, 0, 1, 3, 4, 6]
    m = AllocatorModel(8, 4, order)
    a = m.create()
    m.append(a, 9)                          # 3 blocks
    assert m.table(a) == [5, 2, 7]
    b = m.create()
    m.append(b, 1)
    assert m.table(b) == [0]
    m.free_seq(a)                           # released in logical order: 5, 2, 7
    c = m.create()
    m.append(c, 5)
    assert m.table(c) == [7, 2], "freed blocks come back last-in first-out"
    check_invariants(m)


def test_slots_round_trip_through_cache():
    """Tokens written at their slots and gathered via the table come back in order."""
    rng = np.random.default_rng(3)
    B, NB, Hkv, D = 8, 48, 2, 4
    m = AllocatorModel(NB, B, rng.permutation(NB))
    seqs = [m.create() for _ in range(4)]
    kp = np.full((NB, Hkv, B, D), np.nan, dtype=np.float16)
    vp = kp.copy()
    data = {s: [] for s in seqs}
    for step in range(60):
        s = seqs[rng.integers(4)]
        n = int(rng.integers(1, 6))
        tok = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        slots, pairs = m.append(s, n)
        assert pairs == []
        oc.write_slots(kp, vp, tok, tok, slots, B)
        data[s].extend(tok)
    for s in seqs:
        L = m.length(s)
        got = oc.gather_logical(kp, m.table(s), L, B)
        assert np.array_equal(got, np.array(data[s]).reshape(L, Hkv, D))
    all_slots = [b * B + o for s in seqs for b in m.table(s) for o in range(B)]
    assert len(set(all_slots)) == len(all_slots), "no two requests share a slot"


def test_fork_shares_every_block():
    m = AllocatorModel(16, 4)
    p = m.create()
    m.append(p, 10)
    free_before = len(m.free)
    c = m.fork(p)
    assert m.table(c) == m.table(p) and m.length(c) == 10
    assert len(m.free) == free_before, "fork takes no memory"
    assert all(m.refcount[b] == 2 for b in m.table(p))
    check_invariants(m)


@pytest.mark.parametrize("prompt_len", [64, 65, 100, 127, 128, 512])
def test_parallel_sampling_cow_count(prompt_len):
    """n = 8 samples share the prompt; the first token of each sample copies the
    partly filled last prompt block for 7 of them, the last holder writes in place."""
    B, n = 16, 8
    m = AllocatorModel(400, B)
    p = m.create()
    m.append(p, prompt_len)
    samples = [m.fork(p) for _ in range(n)]
    m.free_seq(p)
    nb = cf.blocks_for_tokens(prompt_len, B)
    assert all(m.refcount[b] == n for b in m.table(samples[0]))
    slots, pairs = m.append_batch(samples)
    partial = prompt_len % B != 0
    assert len(pairs) == (n - 1 if partial else 0)
    assert len({d for _, d in pairs}) == len(pairs)
    # Blocks in use: the shared full prompt blocks + one last block per sample
    # (copied or in place) or one fresh block per sample.
    assert m.stats()["used_blocks"] == ((nb - 1) + n if partial else nb + n)
    for s, slot in zip(samples, slots):
        assert slot // B == m.table(s)[-1]
    check_invariants(m)


def test_cow_keeps_other_readers_view():
    rng = np.random.default_rng(11)
    B, NB, Hkv, D = 4, 16, 1, 2
    m = AllocatorModel(NB, B, rng.permutation(NB))
    kp = np.zeros((NB, Hkv, B, D), dtype=np.float16)
    vp = kp.copy()
    p = m.create()
    prompt = rng.standard_normal((6, Hkv, D)).astype(np.float16)
    oc.write_slots(kp, vp, prompt, prompt, m.append(p, 6)[0], B)
    a, b = m.fork(p), m.fork(p)
    m.free_seq(p)
    view_b = oc.gather_logical(kp, m.table(b), 6, B).copy()
    tok = np.full((1, Hkv, D), 9, dtype=np.float16)
    slots, pairs = m.append(a, 1)
    assert len(pairs) == 1 and pairs[0][0] == m.table(b)[-1]
    oc.copy_blocks([(kp, vp)], pairs)
    oc.write_slots(kp, vp, tok, tok, slots, B)
    assert np.array_equal(oc.gather_logical(kp, m.table(b), 6, B), view_b)
    got_a = oc.gather_logical(kp, m.table(a), 7, B)
    assert np.array_equal(got_a[:6], view_b) and np.array_equal(got_a[6], tok[0])
    # b now holds the last reference: it writes in place.
    slots_b, pairs_b = m.append(b, 1)
    assert pairs_b == [] and slots_b[0] // B == pairs[0][0]


def test_full_shared_block_is_never_written():
    m = AllocatorModel(8, 4)
    p = m.create()
    m.append(p, 8)
    c = m.fork(p)
    slots, pairs = m.append(c, 1)
    assert pairs == [] and slots[0] // 4 not in m.table(p)


def _snapshot(m):
    return copy.deepcopy((m.free, m.refcount, m.tables, m.lengths, m.next_id))


def test_out_of_blocks_changes_nothing():
    m = AllocatorModel(4, 2)
    a = m.create()
    m.append(a, 5)                          # 3 blocks
    b = m.fork(a)
    snap = _snapshot(m)
    with pytest.raises(OutOfBlocks):
        m.append(b, 4)                      # needs 1 CoW + 2 new > 1 free
    assert _snapshot(m) == snap
    with pytest.raises(OutOfBlocks):
        m.append_batch([a, b, a, b])
    assert _snapshot(m) == snap
    with pytest.raises(BadSequence):
        m.append_batch([a, 99])
    assert _snapshot(m) == snap


def test_bad_ids():
    m = AllocatorModel(4, 2)
    a = m.create()
    m.free_seq(a)
    for f in (m.free_seq, m.fork, m.length):
        with pytest.raises(BadSequence):
            f(a)
    with pytest.raises(ValueError):
        AllocatorModel(4, 2, [0, 1, 1, 2])


def _random_ops(m, rng, steps):
    live = []
    epoch = 0
    for _ in range(steps):
        op = rng.integers(7)
        try:
            if op == 0 or not live:
                live.append(m.create())
            elif op == 1:
                live.append(m.fork(live[rng.integers(len(live))]))
            elif op == 2:
                m.append(live[rng.integers(len(live))], int(rng.integers(0, 7)))
            elif op == 3:
                m.append_batch([live[i] for i in rng.integers(len(live), size=3)])
            elif op == 4:
                m.free_seq(live.pop(rng.integers(len(live))))
            elif op == 5:
                epoch += 1
                m.free_seq_deferred(live.pop(rng.integers(len(live))), epoch)
            else:
                m.retire(int(rng.integers(0, epoch + 1)))
        except OutOfBlocks:
            pass
        check_invariants(m)
    m.retire(epoch)
    return live


def test_random_churn_invariants_and_reclamation():
    rng = np.random.default_rng(5)
    for trial in range(20):
        m = AllocatorModel(24, 4, rng.permutation(24))
        live = _random_ops(m, rng, 150)
        for s in live:
            m.free_seq(s)
        check_invariants(m)
        assert len(m.free) == 24 and sum(m.refcount) == 0, "all memory reclaimed"


def test_exhaustive_short_sequences():
    """Every sequence of up to 5 ops from a small alphabet on a 4-block pool."""
    alphabet = ["create", "fork0", "fork_last", "app0_1", "app0_3", "app_last_2", "free0", "batch"]
    for n in range(1, 6):
        for ops in itertools.product(alphabet, repeat=n):
            m = AllocatorModel(4, 2)
            live = []
            for op in ops:
                try:
                    if op == "create":
                        live.append(m.create())
                    elif not live:
                        continue
                    elif op == "fork0":
                        live.append(m.fork(live[0]))
                    elif op == "fork_last":
                        live.append(m.fork(live[-1]))
                    elif op.startswith("app"):
                        who = live[0] if op.startswith("app0") else live[-1]
                        m.append(who, int(op[-1]))
                    elif op == "free0":
                        m.free_seq(live.pop(0))
                    elif op == "batch":
                        m.append_batch(live)
                except OutOfBlocks:
                    pass
                check_invariants(m)
            for s in live:
                m.free_seq(s)
            assert len(m.free) == 4


def test_deferred_free_parks_blocks_until_retired():
    """A block freed at epoch e is not handed out before retire(>= e); then the last
    freed comes back first, as with an immediate free."""
    m = AllocatorModel(6, 4, [0, 1, 2, 3, 4, 5])
    a, b = m.create(), m.create()
    m.append(a, 8)                      # blocks 0, 1
    m.append(b, 4)                      # block 2
    m.free_seq_deferred(a, epoch=1)
    m.free_seq_deferred(b, epoch=2)
    assert m.stats()["pending_blocks"] == 3 and m.stats()["free_blocks"] == 3
    c = m.create()
    m.append(c, 12)                     # must not get 0, 1 or 2
    assert sorted(m.table(c)) == [3, 4, 5]
    with pytest.raises(OutOfBlocks):
        m.append(c, 1)
    assert m.retire(0) == 0
    assert m.retire(1) == 2             # a's blocks, in free order 0 then 1
    assert m.free == [0, 1]
    m.append(c, 1)                      # a fresh block: the last freed, 1
    assert m.table(c)[-1] == 1
    assert m.retire(5) == 1 and m.stats()["pending_blocks"] == 0
    check_invariants(m)
    # a shared block parks only when its last reference goes
    d = m.create()
    m.append(d, 1)
    e = m.fork(d)
    m.free_seq_deferred(d, epoch=9)
    assert m.stats()["pending_blocks"] == 0
    m.free_seq_deferred(e, epoch=10)
    assert m.stats()["pending_blocks"] == 1 and m.parked[0][1] == 10
