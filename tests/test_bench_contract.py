"""The parts of bench.py's contract that need no GPU: a request for more
than one GPU (by flag or by a launcher's WORLD_SIZE), or for the library
comparison outside the linear-layer workload, or for the PyTorch comparison
outside the headline workload, exits at once with a message
and a non-zero status, before torch or the library is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run(["--gpus", n, "--steps", "1", "--warmup", "0"])
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def test_launcher_world_size_is_refused():
    r = _run(["--steps", "1"], {"WORLD_SIZE": "4", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_library_comparison_needs_the_linear_workload():
    r = _run(["--vs-library", "--steps", "1"])
    assert r.returncode == 2 and "--fsdp-linear" in r.stderr and r.stdout == ""


def test_torch_comparison_needs_the_headline_workload():
    for extra in (["--config", "1"], ["--fsdp-linear"]):
        r = _run(["--vs-torch", "--steps", "1", *extra])
        assert r.returncode == 2 and "--vs-torch" in r.stderr and r.stdout == ""
