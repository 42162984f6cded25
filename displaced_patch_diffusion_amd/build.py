"""Builds libdp.so (HIP, gfx950) in-tree with hipcc.

    python -m displaced_patch_diffusion_amd.build

Objects go to _build/ at the repository root; the shared library lands next
to this file so that it travels with the source tree.
"""
from __future__ import annotations

import hashlib
import json
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdp.so")

SOURCES = ["status.cpp", "splice.hip", "groupnorm.hip", "gemm.hip", "attention.hip", "otil.hip"]
# Per-file extra flags.  The attention kernels take finite inputs only, so NaN
# semantics are not kept there: fmax then maps to bare v_max3_f32 without
# per-operand canonicalisation (infinities, used for masking, keep their meaning).
FILE_FLAGS = {"attention.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed-FP32 VALU forms stay disabled for every kernel of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


BUILD_INFO = os.path.join(PKG, "build_info.json")


def source_digest() -> dict:
    """SHA-256 of every library source and header (identifies what a built
    library was compiled from; also recomputed by the benchmark)."""
    out = {}
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            out[name] = hashlib.sha256(f.read()).hexdigest()
    with open(os.path.join(INCLUDE, "dp.h"), "rb") as f:
        out["dp.h"] = hashlib.sha256(f.read()).hexdigest()
    return out


def _git(*args) -> str | None:
    try:
        r = subprocess.run(["git", "-C", ROOT, *args], capture_output=True, text=True, timeout=10)
        return r.stdout.strip() if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def _git_rev() -> str | None:
    """HEAD's revision, suffixed "-dirty" when tracked files differ from it."""
    rev = _git("rev-parse", "HEAD")
    if rev and _git("status", "--porcelain", "--untracked-files=no"):
        rev += "-dirty"
    return rev


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    ver = subprocess.run([HIPCC, "--version"], capture_output=True, text=True).stdout.strip().splitlines()
    info = {"git_rev": _git_rev(), "arch": ARCH, "hipcc": ver[:2], "sources_sha256": source_digest()}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f, indent=1)
    return LIB


if __name__ == "__main__":
    print(build())
