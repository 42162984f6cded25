"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only) and run by oracle/asan_driver.c: every routine on small
shapes with exactly-sized heap buffers, optional arguments given and NULL.
A read or write outside a stated extent, a leak or undefined behaviour fails
the test."""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _gcc(args, cwd):
    return subprocess.run(["gcc", *args], cwd=cwd, capture_output=True, text=True)


def test_oracle_under_asan_and_ubsan(tmp_path):
    probe = tmp_path / "probe.c"
    probe.write_text("int main(void){return 0;}\n")
    if _gcc([*SAN, str(probe), "-o", str(tmp_path / "probe")], tmp_path).returncode != 0:
        pytest.skip("gcc here cannot link the sanitizer runtimes")
    exe = tmp_path / "oracle_asan"
    r = _gcc(["-g", "-O1", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "dp_oracle.c"),
              os.path.join(ROOT, "oracle", "asan_driver.c"), "-o", str(exe), "-lm"], tmp_path)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, OMP_NUM_THREADS="3", ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ran clean" in r.stdout
