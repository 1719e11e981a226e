"""Shared pytest setup.

``gpu`` marks tests that need an MI355X (they call the HIP library through its
C ABI); everything else runs on the CPU.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # A gpu test run without a device is a setup problem, not a pass: fail loudly
    # unless the run explicitly deselected gpu tests.
    pass


def pytest_sessionfinish(session, exitstatus):
    # PKV_MARGINS=<file>: write every attention comparison's margins (test, label,
    # rows, max_abs, rel_l2) as JSON, for the parity-margins summary.
    path = os.environ.get("PKV_MARGINS")
    paths = sys.modules.get("tests.paths")
    if path and paths is not None:
        import json
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump({"exitstatus": int(exitstatus), "margins": paths.MARGINS}, f, indent=0)


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(12345)
