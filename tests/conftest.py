import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP kernels)")


def read_golden(name):
    """Parse a tests/golden/*.txt fixture of 'key: value' lines ('#' starts a comment)."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.strip()
    return out


@pytest.fixture
def golden():
    return read_golden
