"""The multi-step displaced schedule on the GPU (all computation in libdp)
against the oracle's schedule on the same seeded inputs, step by step."""
import numpy as np
import pytest
import torch

import oracle
from displaced_patch_diffusion_amd import schedule, synth
from util import assert_close, host


def say(*a):
    print("case:", *a, flush=True)

pytestmark = pytest.mark.gpu


def _inputs(B, H, W, C, dt, seed=20):
    f = lambda name, shape, std=1.0, mean=0.0: synth.normal(seed, name, shape, std, mean)
    s = C ** -0.5
    raw = {"x0": f("sch.x0", (B, H * W, C)), "wq": f("sch.wq", (C, C), s), "wk": f("sch.wk", (C, C), s),
           "wv": f("sch.wv", (C, C), s), "wo": f("sch.wo", (C, C), s),
           "conv_w": f("sch.cw", (C, 3, 3, C), (9 * C) ** -0.5), "conv_b": f("sch.cb", (C,), 0.1),
           "gamma": f("sch.g", (C,), 0.1, 1.0), "beta": f("sch.b", (C,), 0.1)}
    for k in ("x0", "wq", "wk", "wv", "wo", "conv_w"):
        raw[k] = synth.as_storage(raw[k], dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(t)
    wts = {k: dev(raw[k], tdt) for k in ("wq", "wk", "wv", "wo", "conv_w")}
    wts.update({k: dev(raw[k], torch.float32) for k in ("conv_b", "gamma", "beta")})
    return raw, dev(raw["x0"], tdt), wts


# Multi-step parity runs in float32: a step chains seven rounding points, and
# in bf16 their compounded 1-ulp differences exceed the per-op tolerance (the
# GroupNorm rescales the conv output's rounding by 1/std).  What the schedule
# adds -- which band reads which step's state -- does not depend on the dtype;
# every kernel it calls is checked per op in bf16 elsewhere, and the bf16
# schedule is checked below by its bit-exact stale == fresh property.
@pytest.mark.parametrize("dt,B,H,W,C,heads,N,G,modes,alpha", [
    ("f32", 2, 8, 8, 64, 2, 4, 32, (True, False, False, True, False), 1.0),
    ("f32", 2, 6, 8, 64, 1, 2, 32, (True, False, False), 1.0),  # d = 64
    ("f32", 1, 9, 5, 32, 1, 3, 8, (True, False, False), 1.0),  # 3 bands of 3 rows, d = 32
    ("f32", 2, 8, 8, 64, 2, 4, 32, (True, False, False, False), 0.2),  # sampler update
])
def test_schedule_matches_oracle(dt, B, H, W, C, heads, N, G, modes, alpha):
    say("schedule", dt, B, H, W, C, heads, N, modes)
    raw, x, wts = _inputs(B, H, W, C, dt)
    store = synth.round_to_bf16 if dt == "bf16" else (lambda a: a.astype(np.float32).astype(np.float64))
    ref = oracle.DisplacedSchedule(H, W, heads, N, {k: raw[k] for k in raw if k != "x0"}, G=G,
                                   store=store, store_sums=lambda a: a.astype(np.float32).astype(np.float64))
    gpu = schedule.DisplacedSchedule(H, W, C, heads, N, B, wts, G=G)
    xr = raw["x0"]
    for s, sync in enumerate(modes):
        x = gpu.step(x, sync, alpha)
        xr = ref.step(xr, sync, alpha)
        assert_close(host(x), xr, dt, f"schedule step {s} ({'sync' if sync else 'displaced'})")


def test_schedule_displaced_after_unchanged_input_is_bit_identical():
    """Same input twice: the state recorded by the synchronous step is the
    current state, so the displaced step reproduces it bit for bit."""
    B, H, W, C, heads, N, G = 2, 8, 8, 64, 1, 4, 32
    _, x, wts = _inputs(B, H, W, C, "bf16", seed=21)
    gpu = schedule.DisplacedSchedule(H, W, C, heads, N, B, wts, G=G)
    a = gpu.step(x, True)
    b = gpu.step(x, False)
    assert torch.equal(a, b)
