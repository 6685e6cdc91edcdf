import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes on the CPU oracle)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    """Parse a `key = value` fixture under tests/golden (comment lines start with #)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            try:
                out[k] = int(v)
            except ValueError:
                out[k] = float(v)
    return out
