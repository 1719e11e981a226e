"""bench.py's command line and host-side helpers, on the CPU: more than one GPU is
refused with a message (the benchmark measures one GPU) before anything touches a
device, and no amd-smi child is started under rocprofv3."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert run.returncode == 2
    assert "one GPU" in run.stderr
    assert run.stdout == ""


def test_device_query_skipped_under_profiler(monkeypatch):
    """Under rocprofv3 (which exports ROCPROF_OUTPUT_PATH) gpu_info starts no child."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)

    def refuse(*a, **k):
        raise AssertionError("a child process was started")
    monkeypatch.setattr(subprocess, "run", refuse)
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp")
    assert bench.gpu_info() is None


def test_timing_ring_reads_every_key_once_before_reuse():
    """bench.TimingRing keeps a fixed number of event sets alive and reads each
    set's result before handing it out again, so every key's value survives."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    made = []

    def make():
        made.append([None])
        return made[-1]

    ring = bench.TimingRing(3, make, lambda box: box[0])
    for key in range(10):
        box = ring.take(key)
        box[0] = key * 10                 # the "measurement" of this key
    assert len(made) == 3
    assert ring.results() == {k: k * 10 for k in range(10)}
    assert ring.results() == {k: k * 10 for k in range(10)}    # idempotent
