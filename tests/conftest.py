import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Rows of a |-separated golden file, comments and blank lines skipped."""
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            s = line.strip()
            if not s or s.startswith("#"):
                continue
            rows.append([c.strip() for c in s.split("|")])
    return rows


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
