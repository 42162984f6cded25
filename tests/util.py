"""Helpers shared by the GPU parity tests: device transfer and the tolerances.

Tolerances (written out here, used by every parity test):
  * bf16 outputs: |gpu - oracle| <= 2e-2 elementwise (absolute);
  * f32 outputs:  |gpu - oracle| <= 1e-4 * (|oracle| + rms(oracle)) elementwise,
    i.e. 1e-4 relative with the tensor's rms as the floor for near-zero entries
    (a deliberate choice: an entry far below the rms is a cancellation result
    whose rounding error scales with the terms summed, not with the entry);
    and, with no floor, |gpu - oracle| <= 1e-4 * |oracle| on every entry with
    |oracle| >= rms(oracle) (the largest such ratio is printed per check);
  * the splice: bitwise equality of the whole buffer.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

BF16_ATOL = 2e-2
F32_RTOL = 1e-4


def gpu_ok() -> bool:
    return torch.cuda.is_available()


def torch_dtype(dt: str):
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]


def dev(a: np.ndarray, dt: str) -> torch.Tensor:
    """Exact transfer of bf16/f16/f32-representable float32 values to the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch_dtype(dt)).contiguous()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_violation(gpu: np.ndarray, ref: np.ndarray, dt: str) -> float:
    """Largest |err| / allowed over all elements (<= 1 passes)."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if not np.isfinite(gpu).all():
        return float("inf")
    err = np.abs(gpu - ref)
    if dt == "bf16":
        return float(err.max() / BF16_ATOL) if err.size else 0.0
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    allowed = F32_RTOL * (np.abs(ref) + rms) + 1e-30
    return float((err / allowed).max()) if err.size else 0.0


def max_rel_above_rms(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Largest |gpu - ref| / |ref| over the entries with |ref| >= rms(ref)."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    if not ref.size:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    big = np.abs(ref) >= rms
    if not big.any() or rms == 0.0:
        return 0.0
    return float((np.abs(gpu - ref)[big] / np.abs(ref)[big]).max())


def assert_close(gpu, ref, dt: str, what: str = ""):
    v = max_violation(gpu, ref, dt)
    assert v <= 1.0, f"{what}: tolerance exceeded by factor {v:.3g} ({dt})"
    if dt == "f32":
        r = max_rel_above_rms(gpu, ref)
        print(f"f32 max relative error (|ref| >= rms) {what}: {r:.3g}", file=sys.stderr, flush=True)
        assert r <= F32_RTOL, f"{what}: relative error {r:.3g} above 1e-4 on an entry with |ref| >= rms"
