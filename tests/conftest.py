import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse a tests/golden fixture: '<hex code> <value>' lines, '#' comments."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            code, val = line.split()
            out[int(code, 16)] = float(val)
    return out
