"""Closed forms of the oracle against the values the pages print
(``tests/golden/page_values.json`` holds each value with its citation)."""

import json
import os

import pytest

from oracle import closed_forms as cf

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def test_opt13b_bytes_per_token():
    g = GOLDEN["opt13b_bytes_per_token"]
    assert cf.mha_kv_bytes_per_token(g["hidden"], g["layers"], g["elem_bytes"]) == g["bytes"]
    # 40 heads x 128 = 5120: the grouped form with one KV head per query head agrees.
    assert cf.kv_bytes_per_token(g["layers"], 40, 128, g["elem_bytes"]) == g["bytes"]
    assert g["bytes"] == 800 * 1024


def test_opt13b_request_sizes():
    per_tok = GOLDEN["opt13b_bytes_per_token"]["bytes"]
    g = GOLDEN["opt13b_request_2048_tokens"]
    assert round(g["tokens"] * per_tok / 2 ** 30, 1) == g["printed_gib_one_decimal"]
    g = GOLDEN["opt13b_conversation_2000_tokens"]
    assert g["tokens"] * (per_tok // 1024) / 1e6 == g["printed_million_kb"]


def test_gqa_example_bytes_per_token():
    g = GOLDEN["gqa_example_bytes_per_token"]
    b = cf.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["elem_bytes"])
    assert b == g["bytes"] and b // 1024 == g["printed_kib"]
    s = GOLDEN["gqa_example_sequence_4096"]
    assert b * s["tokens"] // 2 ** 20 == s["printed_mib"]


def test_tail_waste_33_tokens():
    g = GOLDEN["tail_33_tokens"]
    assert cf.blocks_for_tokens(g["tokens"], g["block_size"]) == g["blocks"]
    assert cf.tail_waste_slots(g["tokens"], g["block_size"]) == g["unused_slots"]
    per_tok = GOLDEN[g["bytes_per_token_from"]]["bytes"]
    assert g["unused_slots"] * per_tok / 2 ** 20 == g["printed_mib"]


def test_waste_bound_is_under_one_block():
    g = GOLDEN["max_unused_slots_block16"]
    worst = max(cf.tail_waste_slots(L, g["block_size"]) for L in range(1, 5000))
    assert worst == g["max_unused"]
    for B in (8, 16, 32, 64, 128):
        for L in range(1, 600):
            n = cf.blocks_for_tokens(L, B)
            assert (n - 1) * B < L <= n * B          # the defining property of ceil
            assert 0 <= cf.tail_waste_slots(L, B) < B


def test_block_count_edges():
    assert cf.blocks_for_tokens(0, 16) == 0
    assert [cf.blocks_for_tokens(L, 16) for L in (1, 16, 17, 32, 33)] == [1, 1, 2, 2, 3]
    with pytest.raises(ValueError):
        cf.blocks_for_tokens(-1, 16)
