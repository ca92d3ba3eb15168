import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Parity margins recorded by the GPU tests (what, max |d o|, worst |d o| / bound,
# max |d lse|), printed in the terminal summary so that a quiet (-q) run still
# shows how far inside the tolerance each case sits.
MARGINS = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if not MARGINS:
        return
    tr = terminalreporter
    worst = max(MARGINS, key=lambda m: m[2])
    tr.write_line("parity margins: %d cases; worst |d o|/bound %.3f (%s); max |d o| %.3g; max |d lse| %.3g" % (
        len(MARGINS), worst[2], worst[0], max(m[1] for m in MARGINS), max(m[3] for m in MARGINS)))
    for m in MARGINS:
        if m[0].startswith(("workload", "coverage")):
            tr.write_line("  %-60s |d o| %.3g (%.3f of bound)  |d lse| %.3g" % (m[0][:60], m[1], m[2], m[3]))


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
