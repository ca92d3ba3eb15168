import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """key -> value (str) from a tests/golden/*.txt fixture; '#' lines are comments."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(None, 1)
            out[k] = v
    return out


@pytest.fixture(scope="session")
def golden():
    return read_golden
