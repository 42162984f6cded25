"""dp_groupnorm_stale_stats_noalloc (the library's static device scratch as
workspace) against dp_groupnorm_stale_stats with a workspace of its own: two
calls in a row, the second on a smaller input, then a third in f32.  Both
entry points run the same kernels with the same plan, so outputs and fresh
sums must be bitwise equal."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from displaced_patch_diffusion_amd import ops, synth
from tests.util import dev, dev_f32, gpu_ok

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]


def _case(seed, dt, B, T, C, G, N, rank, silu):
    x = dev(synth.random_tensor(seed, "na.x", (B, T, C), dt, 1.3), dt)
    stale = dev_f32(np.abs(synth.random_tensor(seed, "na.s", (N, B, G, 2), "f32", 50.0)))
    gamma = dev_f32(synth.random_tensor(seed, "na.g", (C,), "f32", 1.0))
    beta = dev_f32(synth.random_tensor(seed, "na.b", (C,), "f32", 1.0))
    return x, stale, gamma, beta


@pytest.mark.parametrize("calls", [[("bf16", 2, 7200, 640, 32, 4, 1, True), ("bf16", 1, 1000, 128, 32, 2, 0, False),
                                    ("f32", 3, 333, 64, 8, 3, 2, True)]])
def test_noalloc_matches_workspace_entry(calls):
    for i, (dt, B, T, C, G, N, rank, silu) in enumerate(calls):
        print(f"no-alloc call {i}: {dt} B={B} T={T} C={C} G={G} N={N} rank={rank} silu={silu}",
              file=sys.stderr, flush=True)
        x, stale, gamma, beta = _case(10 + i, dt, B, T, C, G, N, rank, silu)
        T_total = N * T
        y_ref, y = torch.empty_like(x), torch.full_like(x, float("nan"))
        f_ref = torch.empty((B, G, 2), dtype=torch.float32, device="cuda")
        f = torch.full_like(f_ref, float("nan"))
        ops.dp_groupnorm_stale_stats(x, stale, rank, T_total, gamma, beta, 1e-5, silu, G, y=y_ref,
                                     fresh_sums_out=f_ref)
        ops.dp_groupnorm_stale_stats_noalloc(x, stale, rank, T_total, gamma, beta, 1e-5, silu, G, y,
                                             fresh_sums_out=f)
        torch.cuda.synchronize()
        assert torch.equal(f, f_ref), f"call {i}: fresh sums differ"
        assert torch.equal(y, y_ref), f"call {i}: outputs differ"


def test_noalloc_replays_in_a_hip_graph():
    """The callers it is for: the call captured in a HIP graph (after one
    eager call, which does the per-device set-up) and replayed three times
    with eager work in between; every replay equals the workspace entry
    point's output."""
    dt, B, T, C, G, N, rank = "bf16", 2, 2000, 320, 32, 4, 2
    print(f"no-alloc graph: {dt} B={B} T={T} C={C} G={G}", file=sys.stderr, flush=True)
    x, stale, gamma, beta = _case(20, dt, B, T, C, G, N, rank, True)
    y_ref = torch.empty_like(x)
    f_ref = torch.empty((B, G, 2), dtype=torch.float32, device="cuda")
    ops.dp_groupnorm_stale_stats(x, stale, rank, N * T, gamma, beta, 1e-5, True, G, y=y_ref, fresh_sums_out=f_ref)
    y, f = torch.empty_like(x), torch.empty_like(f_ref)
    ops.dp_groupnorm_stale_stats_noalloc(x, stale, rank, N * T, gamma, beta, 1e-5, True, G, y, fresh_sums_out=f)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.dp_groupnorm_stale_stats_noalloc(x, stale, rank, N * T, gamma, beta, 1e-5, True, G, y, fresh_sums_out=f)
    torch.cuda.synchronize()
    for i in range(3):
        y.fill_(float("nan"))
        f.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(f, f_ref), f"replay {i}: fresh sums differ"
        assert torch.equal(y, y_ref), f"replay {i}: outputs differ"
