"""bench.py's command-line contract on the host: more than one GPU is refused
with a message before anything touches a device, and without a GPU the
script stops with its own message instead of a traceback."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = _run("--gpus", n)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout.strip() == ""


def test_no_gpu_stops_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0", "--cpu-seconds", "0")
    assert r.returncode == 1 and "needs a GPU" in r.stderr
    assert "Traceback" not in r.stderr
