import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")


def read_golden(name):
    """Rows of a golden file as lists of whitespace-separated fields (comments dropped)."""
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def half_ulp(printed: str) -> float:
    """Half a unit of the last printed digit of a decimal string."""
    if "." in printed:
        return 0.5 * 10.0 ** (-len(printed.split(".")[1]))
    return 0.5


@pytest.fixture
def golden():
    return read_golden
