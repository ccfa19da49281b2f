import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def read_golden_rows(name):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def golden_constants():
    out = {}
    for r in read_golden_rows("constants.txt"):
        out[r[0]] = float(r[1])
    return out
