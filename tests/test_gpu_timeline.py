"""The instrumented library (libpagedkv_timeline.so) records one timeline entry per
streaming wave of a decode launch: `bench.py --timeline` on the GQA workload, in a
process of its own so that only the instrumented library is loaded there."""

import os
import re
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_timeline_records_every_wave_of_the_launch():
    lib = os.path.join(ROOT, "paged_kv_cache_244_amd", "libpagedkv_timeline.so")
    if not os.path.exists(lib):
        pytest.fail("libpagedkv_timeline.so is not built (run __graft_entry__.build())")
    print("timeline: bench.py --workload gqa --timeline --warmup 2 --replicas 1", flush=True)
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "gqa",
                          "--timeline", "--warmup", "2", "--replicas", "1"],
                         capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stderr[-3000:]
    text = run.stdout
    items = int(re.search(r"'num_items': (\d+)", text).group(1))
    waves = int(re.search(r"^waves (\d+), launch span ([\d.]+) us", text, re.M).group(1))
    span = float(re.search(r"^waves \d+, launch span ([\d.]+) us", text, re.M).group(1))
    # GQA 32/8 on the MFMA kernel: 8 head tiles of 4 query heads per work-list entry,
    # and every piece of a plain decode streams tokens.
    assert waves == items * 8
    assert 0 < span < 10_000
    assert "resident waves every 2 us" in text and "XCD" in text


def test_prefill_timeline_records_tile_pairs():
    lib = os.path.join(ROOT, "paged_kv_cache_244_amd", "libpagedkv_timeline.so")
    if not os.path.exists(lib):
        pytest.fail("libpagedkv_timeline.so is not built (run __graft_entry__.build())")
    print("timeline: bench.py --workload prefill --timeline --warmup 2", flush=True)
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "prefill",
                          "--timeline", "--warmup", "2"], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stderr[-3000:]
    text = run.stdout
    waves, groups = (int(x) for x in re.search(r"(\d+) waves of (\d+) full workgroups", text).groups())
    assert groups > 0 and waves == 8 * groups
    pair = float(re.search(r"^pair: ([\d.]+) cycles", text, re.M).group(1))
    assert 1000 < pair < 100_000
