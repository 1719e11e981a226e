"""Pins of the oracle's table check (oracle.cache.check_tables): hand-worked cases
and a second, vectorised formulation of the same definition on random tables."""
import numpy as np

from oracle import cache as oc

TABLES = [[3, 4, 99], [0, -1, 7]]


def test_entries_past_the_context_are_not_checked():
    # 20 tokens need 2 blocks (3, 4); 16 tokens need 1 block (0): 99, -1 and 7 lie past.
    assert oc.check_tables(TABLES, [20, 16], 16, 10) == (0, 0, -1, -1)


def test_id_faults_and_the_first_offender():
    # 33 tokens reach entry 2 (99 >= 10); 17 tokens reach entry 1 (-1).
    assert oc.check_tables(TABLES, [33, 17], 16, 10) == (2, 0, 0, 2)
    # Request 0 clean (3 < 5); request 1 needs 3 entries: -1 and 7 are outside 5 blocks.
    assert oc.check_tables(TABLES, [16, 48], 16, 5) == (2, 0, 1, 1)


def test_length_faults():
    # A negative length is a fault and covers nothing; 49 tokens need 4 > 3 blocks,
    # and its 3 entries are still checked (-1 is outside).  Request 0's length comes first.
    assert oc.check_tables(TABLES, [-5, 49], 16, 10) == (1, 2, 0, -1)
    # A row of width 0 holds no context but the empty one.
    assert oc.check_tables(np.zeros((2, 0), np.int32), [0, 1], 16, 10) == (0, 1, 1, -1)


def test_empty_contexts_and_empty_pool():
    assert oc.check_tables(TABLES, [0, 0], 16, 10) == (0, 0, -1, -1)
    assert oc.check_tables(TABLES, [16, 1], 16, 0) == (2, 0, 0, 0)
    assert oc.check_tables(np.zeros((0, 4), np.int32), [], 16, 10) == (0, 0, -1, -1)


def test_agrees_with_a_vectorised_count():
    rng = np.random.default_rng(5)
    for _ in range(200):
        s, mb, bs, nb = rng.integers(1, 9), rng.integers(0, 12), int(rng.choice([8, 16, 32])), rng.integers(0, 50)
        tables = rng.integers(-3, nb + 3, size=(s, mb)).astype(np.int32)
        lens = rng.integers(-20, mb * bs + 40, size=s).astype(np.int32)
        needed = np.where(lens < 0, 0, -(-lens // bs))
        covered = np.arange(mb)[None, :] < np.minimum(needed, mb)[:, None]
        bad = covered & ((tables < 0) | (tables >= nb))
        len_bad = (lens < 0) | (needed > mb)
        got = oc.check_tables(tables, lens, bs, nb)
        assert got[:2] == (int(bad.sum()), int(len_bad.sum()))
        keys = [(r, -1) for r in np.flatnonzero(len_bad)] + [tuple(x) for x in np.argwhere(bad)]
        assert got[2:] == (min(keys) if keys else (-1, -1))
