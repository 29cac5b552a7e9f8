"""bench.py's command-line contract on a host without a GPU: one GPU only (any other --gpus exits
with a message and status 2), and the long-context options are checked before anything runs."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_help_lists_the_workload_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--config", "--r", "--seq", "--tokens", "--loss-side", "--no-loss-side", "--steps", "--warmup"):
        assert opt in r.stdout
