"""bench.py on more than one GPU: refused with a message (this build measures one
GPU), before anything touches a device.  Runs on the CPU."""

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
