"""The library driven through its C ABI alone: ``tests/c_abi_decode.cpp`` (built by
``build()``) is host C++ linked against libpagedkv.so and the HIP runtime, with no
Python or torch between the caller and the library.  It reserves slots with the
host allocator (a fork whose append copies a shared, partly filled block), writes
and copies K/V, and runs pa_decode in one pass and in 16-token partitions; it checks
the bytes bit for bit and the outputs against exact properties (one token: its V;
equal keys: the mean of V)."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_decode")


def test_c_abi_decode_program():
    if not os.path.exists(EXE):
        pytest.fail("tests/c_abi_decode is not built: run __graft_entry__.build()")
    print("\n[case] c_abi_decode (C ABI only)", flush=True)
    run = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "c_abi_decode OK" in run.stdout, (run.stdout, run.stderr)
