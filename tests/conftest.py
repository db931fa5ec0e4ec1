import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-only test, skipped unless --runslow")


def pytest_addoption(parser):
    parser.addoption("--runslow", action="store_true", default=False, help="run slow CPU tests")


def pytest_collection_modifyitems(config, items):
    if config.getoption("--runslow"):
        return
    skip = pytest.mark.skip(reason="slow tier: pass --runslow")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)


def golden(name):
    """Parse a whitespace table under tests/golden/ (comments start with #)."""
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def golden_dict(name):
    out = {}
    for row in golden(name):
        vals = [[float(v) for v in col.split(",")] for col in row[1:]]
        out[row[0]] = vals
    return out
