import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


_TIMES = os.environ.get("CPTHD_TEST_TIMES")


def pytest_runtest_logreport(report):
    """With CPTHD_TEST_TIMES naming a file, append each test's outcome and wall time (set-up + call) as it ends."""
    if _TIMES and report.when in ("setup", "call"):
        with open(_TIMES, "a") as f:
            f.write(f"{report.when}\t{report.outcome}\t{report.duration:.2f}\t{report.nodeid}\n")
