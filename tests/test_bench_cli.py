"""bench.py's command-line contract that needs no GPU: one GPU only, and an
unknown workload is rejected before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env)


def test_more_than_one_gpu_exits_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "ONE GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_exits_with_a_message():
    env = dict(os.environ, WORLD_SIZE="2")
    r = run("--gpus", "1", env=env)
    assert r.returncode == 2 and "WORLD_SIZE=2" in r.stderr
