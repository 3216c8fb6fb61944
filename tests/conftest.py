import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes)")


def pytest_collection_modifyitems(config, items):
    # Full-size workloads run late so that a failure there hides nothing else; the
    # allocation-free entry point's file runs after everything.
    def order(it):
        if os.path.basename(str(it.fspath)).startswith("test_zz_"):
            return 2
        return 1 if it.get_closest_marker("slow") else 0

    items.sort(key=order)


def pytest_runtest_logstart(nodeid, location):
    # On GPU runs, name each case in a progress file before it starts, so that a
    # run cut short still says which case was running.
    path = os.environ.get("MSA_PROGRESS_LOG")
    if path:
        with open(path, "a") as f:
            f.write(nodeid + "\n")
            f.flush()
