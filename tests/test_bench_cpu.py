"""Host-side contract of bench.py (no GPU needed): it measures the one-GPU
path only, so a request for more GPUs exits with a message and status 2
before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one-GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run("--steps", "1", "--warmup", "0", env=env)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr


def test_help_documents_the_step():
    r = _run("--help")
    assert r.returncode == 0
    assert "verify block" in r.stdout and "--budget-sweep" in r.stdout
