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


def test_rank_outside_the_workload_is_rejected():
    r = run("--rank", "9")
    assert r.returncode != 0 and "--rank must be in [0, 8)" in r.stderr


def test_stream_salt_selects_other_streams_and_zero_restores_them():
    from displaced_patch_diffusion_amd import synth

    base = synth.normal(1, "salt.check", (8,))
    try:
        synth.set_stream_salt(3)
        other = synth.normal(1, "salt.check", (8,))
    finally:
        synth.set_stream_salt(0)
    assert not (other == base).all()
    assert (synth.normal(1, "salt.check", (8,)) == base).all()
