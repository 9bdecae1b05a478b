import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def read_golden(name):
    """Parse a tests/golden fixture: '# comments', 'key = ints' lines."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            vals = [int(x) for x in v.split()]
            out.setdefault(k.strip(), []).append(vals)
    return out
