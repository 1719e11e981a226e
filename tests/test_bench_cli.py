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
