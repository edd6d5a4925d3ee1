"""bench.py's command line on a machine without a GPU: more than one GPU is
refused with a message, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_distributed_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = _run("--gpus", "1", env=env)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
