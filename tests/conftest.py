import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """key = value lines; '#' starts a comment."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (x.strip() for x in line.split("=", 1))
            out[k] = float(v)
    return out


@pytest.fixture(scope="session")
def oracle_lib():
    from oracle import _c
    return _c.lib()
