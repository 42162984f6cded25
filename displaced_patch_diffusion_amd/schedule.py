"""Multi-step displaced schedule on one GPU.

N row bands of one layer stack -- attention block (projections, K/V splice,
attention, output projection), 3x3 conv with halo rows, GroupNorm -- stepped
through several denoising steps, each step's output feeding the next.  Method
source: the DistriFusion project summary, "How It Works" (a synchronous step,
then steps that reuse the activations the other devices produced one step
earlier, exchanged asynchronously) and "OTIL for SDXL on 4x L40S", "What is
implemented where" (the displaced state: K/V buffers, conv halo rows, two
GroupNorm scalars per group).

A synchronous step gives every band the current step's K/V rows, halo rows
and group sums of all bands.  A displaced step gives band r its own fresh
values and the other bands' values recorded during the previous step.  The
bands run one after another on one stream; what a multi-GPU run would
exchange over the interconnect is a device copy here:
  * K/V: every band splices its fresh rows into this step's full buffers
    (an all-gather); a displaced band attends over the previous step's
    buffers with its own rows spliced in, then restores them;
  * halo rows: copies of the neighbours' attention-block output rows;
  * group sums: each band's fresh [B, G, 2] sums.
Every computation of the layer stack runs in the libdp kernels; torch
provides memory, copies and the stream, and the synthetic sampler update
x <- x + alpha (stack(x) - x) between steps (one lerp; alpha = 1 feeds the
stack's output straight to the next step).  With alpha < 1 consecutive steps'
activations stay close, as along a diffusion trajectory, which is what makes
the previous step's state a usable stand-in.
"""
from __future__ import annotations

import argparse
import json
import time

import torch

from . import ops
from .partition import row_bands


class DisplacedSchedule:
    def __init__(self, H: int, W: int, C: int, heads: int, N: int, B: int, weights: dict,
                 G: int = 32, eps: float = 1e-5):
        self.H, self.W, self.C, self.heads, self.N, self.B, self.G, self.eps = H, W, C, heads, N, B, G, eps
        self.w = weights
        dt = weights["wq"].dtype
        dev = weights["wq"].device
        self.bands = row_bands(H, N)
        T = H * W

        def buf(*shape, dtype=dt):
            return torch.empty(shape, dtype=dtype, device=dev)

        self.k = [buf(B, T, C), buf(B, T, C)]  # [this step, previous step]
        self.v = [buf(B, T, C), buf(B, T, C)]
        self.sums = [buf(N, B, G, 2, dtype=torch.float32), buf(N, B, G, 2, dtype=torch.float32)]
        self.band = []
        for r0, r1 in self.bands:
            Tr = (r1 - r0) * W
            self.band.append({
                "x": buf(B, Tr, C), "q": buf(B, Tr, C), "kf": buf(B, Tr, C), "vf": buf(B, Tr, C),
                "o": buf(B, Tr, C), "y": [buf(B, Tr, C), buf(B, Tr, C)], "z": buf(B, Tr, C),
                "out": buf(B, Tr, C), "ks": buf(B, Tr, C), "vs": buf(B, Tr, C),
                "top": buf(B, W, C), "bot": buf(B, W, C),
            })
        heights = sorted({r1 - r0 for r0, r1 in self.bands})
        Tq_max = heights[-1] * W
        attn_bytes = max(ops.dp_attn_stale_kv_workspace(B, heads, h * W, T, C // heads, dt) for h in heights)
        self.attn_ws = torch.empty(max(1, attn_bytes), dtype=torch.uint8, device=dev)
        self.gn_ws = torch.zeros(ops.dp_groupnorm_stale_stats_workspace(B, Tq_max, C, G),
                                 dtype=torch.uint8, device=dev)
        self.cur = 0
        self.has_prev = False

    def step(self, x: torch.Tensor, sync: bool, alpha: float = 1.0) -> torch.Tensor:
        """x [B, H*W, C] -> x + alpha (stack(x) - x); records this step's state."""
        if not sync and not self.has_prev:
            raise ValueError("a displaced step needs a previous step")
        w, W, B, C = self.w, self.W, self.B, self.C
        cur, prev = self.cur, 1 - self.cur
        kc, vc, kp, vp = self.k[cur], self.v[cur], self.k[prev], self.v[prev]
        # projections; this step's full K/V buffers (the exchange)
        for (r0, r1), s in zip(self.bands, self.band):
            s["x"].copy_(x[:, r0 * W:r1 * W])
            ops.dp_linear(s["x"], w["wq"], y=s["q"])
            ops.dp_linear(s["x"], w["wk"], y=s["kf"])
            ops.dp_linear(s["x"], w["wv"], y=s["vf"])
            ops.dp_kv_buffer_splice(kc, vc, s["kf"], s["vf"], r0 * W)
        # attention over the current (sync) or previous step's buffers
        for (r0, r1), s in zip(self.bands, self.band):
            if sync:
                ops.dp_attn_stale_kv(s["q"], kc, vc, self.heads, out=s["o"], ws=self.attn_ws)
            else:
                s["ks"].copy_(kp[:, r0 * W:r1 * W])
                s["vs"].copy_(vp[:, r0 * W:r1 * W])
                ops.dp_kv_buffer_splice(kp, vp, s["kf"], s["vf"], r0 * W)
                ops.dp_attn_stale_kv(s["q"], kp, vp, self.heads, out=s["o"], ws=self.attn_ws)
                ops.dp_kv_buffer_splice(kp, vp, s["ks"], s["vs"], r0 * W)
            ops.dp_linear(s["o"], w["wo"], y=s["y"][cur])
        # conv with the neighbours' rows of this step (sync) or the previous one
        src = cur if sync else prev
        for r, ((r0, r1), s) in enumerate(zip(self.bands, self.band)):
            h = r1 - r0
            top = bot = None
            if r0 > 0:
                top = s["top"]
                top.copy_(self.band[r - 1]["y"][src].view(B, -1, W, C)[:, -1])
            if r1 < self.H:
                bot = s["bot"]
                bot.copy_(self.band[r + 1]["y"][src].view(B, -1, W, C)[:, 0])
            ops.dp_conv3x3_stale_halo(s["y"][cur].view(B, h, W, C), top, bot, w["conv_w"], w["conv_b"],
                                      y=s["z"].view(B, h, W, C))
        # GroupNorm with every band's sums of this step (sync) or the previous one
        if sync:
            for r, ((r0, r1), s) in enumerate(zip(self.bands, self.band)):
                ops.dp_groupnorm_stale_stats(s["z"], None, 0, (r1 - r0) * W, None, None, self.eps, False,
                                             self.G, y=s["out"], fresh_sums_out=self.sums[cur][r],
                                             ws=self.gn_ws)
            stale = self.sums[cur]
        else:
            stale = self.sums[prev]
        x_next = torch.empty_like(x)
        for r, ((r0, r1), s) in enumerate(zip(self.bands, self.band)):
            ops.dp_groupnorm_stale_stats(s["z"], stale, r, self.H * W, w["gamma"], w["beta"], self.eps,
                                         False, self.G, y=s["out"],
                                         fresh_sums_out=None if sync else self.sums[cur][r], ws=self.gn_ws)
            x_next[:, r0 * W:r1 * W].copy_(s["out"])
        if alpha != 1.0:
            x_next = torch.lerp(x, x_next, alpha)
        self.cur = prev
        self.has_prev = True
        return x_next


def is_sync(s: int, warmup: int, refresh: int) -> bool:
    """Steps before `warmup` are synchronous, and so is every `refresh`-th
    step after them (0: never again)."""
    return s < warmup or (refresh > 0 and (s - warmup) % refresh == refresh - 1)


def _device_inputs(w, dev):
    from . import synth  # seeded generator only
    raw = synth.schedule_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    to = lambda a, t: torch.from_numpy(a.astype("float32")).to(dev).to(t).contiguous()
    weights = {k: to(raw[k], dt) for k in ("wq", "wk", "wv", "wo", "conv_w")}
    weights.update({k: to(raw[k], torch.float32) for k in ("conv_b", "gamma", "beta")})
    return to(raw["x0"], dt), weights


def main() -> None:
    """Drift of the displaced schedule against the all-synchronous one, and
    the time per step of both, on a single-level workload."""
    from . import synth
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="sdxl3840_l240_c640")
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--refresh", type=int, default=0)
    ap.add_argument("--alpha", type=float, default=0.1)
    args = ap.parse_args()
    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda")
    x0, weights = _device_inputs(w, dev)
    runs = {}
    for name in ("sync", "displaced"):
        sch = DisplacedSchedule(w.attn_H, w.attn_W, w.attn_C, w.heads, w.N, w.B, weights, w.G, w.eps)
        x = x0
        xs, times = [], []
        for s in range(args.steps):
            sync = name == "sync" or is_sync(s, args.warmup, args.refresh)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            x = sch.step(x, sync, args.alpha)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
            xs.append(x.float())
        runs[name] = (xs, times)
    drift = [float((a - b).norm() / b.norm()) for a, b in zip(runs["displaced"][0], runs["sync"][0])]
    ms = {k: 1e3 * sum(v[1][1:]) / max(1, len(v[1]) - 1) for k, v in runs.items()}
    print(json.dumps({"workload": args.workload, "n_patches": w.N, "steps": args.steps,
                      "warmup": args.warmup, "refresh": args.refresh, "alpha": args.alpha,
                      "ms_per_step": ms, "relative_drift_per_step": drift}))


if __name__ == "__main__":
    main()
