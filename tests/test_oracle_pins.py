"""The CPU oracle against facts fixed outside it (closed forms, a library routine,
brute force, invariants).  See ``oracle_pins.py`` for what each pin checks."""

import types

import numpy as np
import pytest

import oracle
from tests import oracle_pins

IMPL = types.SimpleNamespace(
    attend_one=oracle.attention.attend_one,
    attend_paged=oracle.attention.attend_paged,
    attend_contiguous=oracle.attention.attend_contiguous,
    attend_prefill_paged=oracle.attention.attend_prefill_paged,
    gather_logical=oracle.cache.gather_logical,
    write_slots=oracle.cache.write_slots,
    copy_blocks=oracle.cache.copy_blocks,
)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(IMPL, np.random.default_rng(7))
