import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host work)")


def read_golden_ints(name):
    """Like read_golden, with integer values kept exact."""
    rows = {}
    with open(os.path.join(TESTS, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                rows[k] = int(v)
    return rows


def read_golden(name):
    """Parse a tests/golden fixture: '#' comments, then 'key value' lines."""
    rows = {}
    with open(os.path.join(TESTS, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                rows[k] = float(v)
    return rows
