import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU statistics test")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


def read_golden(name):
    """Parse a tests/golden fixture: '# ...' comments, 'key = value' lines."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = [s.strip() for s in line.split("=", 1)]
            out[k] = v
    return out


def floats(s):
    return [[float(x) for x in part.split()] for part in s.split("|")]


def ints(s):
    return [int(x) for x in s.split()]
