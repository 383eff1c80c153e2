"""The C ABI without Python: tests/capi_demo (built by build()) allocates
with hipMalloc, runs three fused steps and gathers of one ZeRO-3 rank on a
ragged three-unit layout, and compares master, m, v and the full bf16
buffer bit for bit with the C oracle on the same inputs."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "capi_demo")


def test_c_program_matches_the_oracle():
    if not os.path.exists(DEMO):
        # a host-only gcc build (seconds) against the already built libraries
        import sys
        sys.path.insert(0, ROOT)
        import __graft_entry__
        __graft_entry__.build_capi_demo()
    assert os.path.exists(DEMO)
    r = subprocess.run([DEMO], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "capi demo ok" in r.stdout and "bit-exact" in r.stdout
