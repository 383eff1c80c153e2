import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# test_mutants_oracle.py runs the oracle's pins in a child process against a
# copy of oracle/ with one planted mistake; this variable names the folder
# holding that copy, so `import oracle` finds it before the real one.
_MUTANT_ROOT = os.environ.get("ZS_ORACLE_MUTANT_ROOT")
if _MUTANT_ROOT:
    sys.path.insert(0, _MUTANT_ROOT)

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
