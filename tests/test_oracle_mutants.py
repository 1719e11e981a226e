"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
at least one pin catches each: evidence the pins constrain every term."""

import types

import numpy as np
import pytest

import oracle
from tests import oracle_pins


def _attend_factory(head_map=None, subtract_max=True, use_scale=True, normalise=True,
                    transpose_values=False, sign=1.0):
    def attend_one(q_heads, keys, values, scale):
        q_heads = np.asarray(q_heads, dtype=np.float64)
        keys = np.asarray(keys, dtype=np.float64)
        values = np.asarray(values, dtype=np.float64)
        Hq, D = q_heads.shape
        L, Hkv, _ = keys.shape
        out = np.zeros((Hq, D))
        if L == 0:
            return out
        G = Hq // Hkv
        s64 = np.float64(np.float32(scale)) if use_scale else 1.0
        for h in range(Hq):
            g = head_map(h, Hq, Hkv) if head_map else h // G
            sc = sign * s64 * (keys[:, g, :] @ q_heads[h])
            w = np.exp(sc - sc.max()) if subtract_max else np.exp(sc)
            p = w / w.sum() if normalise else w
            vals = values[:, g, :]
            if transpose_values:
                vals = vals[::-1]
            out[h] = p @ vals
        return out
    return attend_one


def _gather_wrong_offset(pool, table_row, num_tokens, block_size):
    t = np.arange(num_tokens)
    phys = np.asarray(table_row)[t // block_size]
    return pool[phys, :, (t + 1) % block_size, :]


def _gather_contiguous_ignoring_table(pool, table_row, num_tokens, block_size):
    t = np.arange(num_tokens)
    return pool[t // block_size, :, t % block_size, :]


def _write_swapped(k_pool, v_pool, k_new, v_new, slot_mapping, block_size):
    for j, s in enumerate(slot_mapping):
        if s < 0:
            continue
        k_pool[s % k_pool.shape[0], :, s // k_pool.shape[0] % block_size, :] = k_new[j]
        v_pool[s % k_pool.shape[0], :, s // k_pool.shape[0] % block_size, :] = v_new[j]
    return k_pool, v_pool


def _write_kv_crossed(k_pool, v_pool, k_new, v_new, slot_mapping, block_size):
    return oracle.cache.write_slots(k_pool, v_pool, v_new, k_new, slot_mapping, block_size)


def _copy_backwards(layer_pools, block_pairs):
    return oracle.cache.copy_blocks(layer_pools, [(d, s) for s, d in block_pairs])


def _copy_first_layer_only(layer_pools, block_pairs):
    oracle.cache.copy_blocks(layer_pools[:1], block_pairs)
    return layer_pools


def _attend_paged_with(attend_one, gather=oracle.cache.gather_logical):
    def attend_paged(q, k_pool, v_pool, block_tables, context_lens, block_size, scale, seqs=None):
        q = np.asarray(q)
        out = np.zeros(q.shape)
        for i in range(q.shape[0]) if seqs is None else seqs:
            L = int(context_lens[i])
            out[i] = attend_one(q[i], gather(k_pool, block_tables[i], L, block_size),
                                gather(v_pool, block_tables[i], L, block_size), scale)
        return out
    return attend_paged


def _impl(**over):
    base = dict(
        attend_one=oracle.attention.attend_one,
        attend_paged=oracle.attention.attend_paged,
        attend_contiguous=oracle.attention.attend_contiguous,
        attend_prefill_paged=oracle.attention.attend_prefill_paged,
        gather_logical=oracle.cache.gather_logical,
        write_slots=oracle.cache.write_slots,
        copy_blocks=oracle.cache.copy_blocks,
    )
    base.update(over)
    if "attend_one" in over and "attend_paged" not in over:
        base["attend_paged"] = _attend_paged_with(over["attend_one"])
    if "gather_logical" in over:
        base["attend_paged"] = _attend_paged_with(base["attend_one"], over["gather_logical"])
    return types.SimpleNamespace(**base)


def _contiguous_factory(extra_token=0, swap=True):
    def attend_contiguous(q, k_rows, v_rows, context_lens, scale, seqs=None):
        q = np.asarray(q)
        out = np.zeros(q.shape, dtype=np.float64)
        for i in range(q.shape[0]):
            n = int(context_lens[i]) + extra_token
            k, v = k_rows[i, :, :n, :], v_rows[i, :, :n, :]
            if swap:
                k, v = np.swapaxes(k, 0, 1), np.swapaxes(v, 0, 1)
            out[i] = oracle.attention.attend_one(q[i], k, v, scale)
        return out
    return attend_contiguous


def _prefill_factory(see_ahead=0, from_start=False):
    def attend_prefill_paged(q, k_pool, v_pool, block_tables, context_lens, q_starts, block_size,
                             scale):
        q = np.asarray(q)
        out = np.zeros(q.shape, dtype=np.float64)
        for i in range(len(context_lens)):
            L = int(context_lens[i])
            first, last = int(q_starts[i]), int(q_starts[i + 1])
            keys = oracle.cache.gather_logical(k_pool, block_tables[i], L, block_size)
            vals = oracle.cache.gather_logical(v_pool, block_tables[i], L, block_size)
            for j in range(last - first):
                pos = j if from_start else L - (last - first) + j
                n = min(L, pos + 1 + see_ahead)
                out[first + j] = oracle.attention.attend_one(q[first + j], keys[:n], vals[:n], scale)
        return out
    return attend_prefill_paged


MUTANTS = {
    "prefill_sees_next_token": _impl(attend_prefill_paged=_prefill_factory(see_ahead=1)),
    "prefill_positions_from_zero": _impl(attend_prefill_paged=_prefill_factory(from_start=True)),
    "rows_read_one_past_length": _impl(attend_contiguous=_contiguous_factory(extra_token=1)),
    "rows_axes_not_swapped": _impl(attend_contiguous=_contiguous_factory(swap=False)),
    "head_map_modulo": _impl(attend_one=_attend_factory(head_map=lambda h, Hq, Hkv: h % Hkv)),
    "no_max_subtraction_overflow": _impl(attend_one=_attend_factory(subtract_max=False)),
    "scale_dropped": _impl(attend_one=_attend_factory(use_scale=False)),
    "not_normalised": _impl(attend_one=_attend_factory(normalise=False)),
    "values_reversed": _impl(attend_one=_attend_factory(transpose_values=True)),
    "score_sign_flipped": _impl(attend_one=_attend_factory(sign=-1.0)),
    "gather_offset_off_by_one": _impl(gather_logical=_gather_wrong_offset),
    "gather_ignores_table": _impl(gather_logical=_gather_contiguous_ignoring_table),
    "write_block_offset_swapped": _impl(write_slots=_write_swapped),
    "write_k_v_crossed": _impl(write_slots=_write_kv_crossed),
    "copy_direction_reversed": _impl(copy_blocks=_copy_backwards),
    "copy_one_layer_only": _impl(copy_blocks=_copy_first_layer_only),
}


def _caught(impl):
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl, np.random.default_rng(7))
        except (AssertionError, FloatingPointError, IndexError, ValueError, ZeroDivisionError):
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert _caught(MUTANTS[name]) is not None, f"no pin catches mutant {name}"
