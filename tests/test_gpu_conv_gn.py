"""Conv with GroupNorm sums in its epilogue, and GroupNorm from given sums.

dp_conv3x3_stale_halo_gn_sums must write exactly dp_conv3x3_stale_halo's y
and sums equal to the oracle's group sums of that y (float32 accumulation:
within 2e-5 of sum|y| and of sum y^2), over tiles that end at batch edges,
tiles that straddle them and every tile shape; dp_groupnorm_apply with the
sums dp_groupnorm_sums returns must equal dp_groupnorm_stale_stats bit for
bit; workspaces reused across calls and shapes keep working (the conv's
needs no initial contents).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from displaced_patch_diffusion_amd import ops, synth
from tests.util import dev, dev_f32, gpu_ok, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]
R = synth.random_tensor


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def check_sums(g, y, G):
    ref = oracle.group_sums(y, G)
    B, T, C = y.shape
    ya = np.abs(y).reshape(B, T, G, C // G).sum(axis=(1, 3))
    assert np.all(np.abs(g[..., 0] - ref[..., 0]) <= 2e-5 * ya + 1e-6)
    assert np.all(np.abs(g[..., 1] - ref[..., 1]) <= 2e-5 * ref[..., 1] + 1e-6)


@pytest.mark.parametrize("B,h,W,Cin,Cout,G,halos", [
    (2, 30, 240, 640, 640, 32, "both"),   # the SDXL-3840 share (160x128 tiles, tiles end at batch edges)
    (2, 13, 100, 64, 160, 32, "top"),     # tiles straddle the batch boundary
    (3, 7, 50, 64, 64, 8, "bottom"),      # small: 64x64 tiles, three batch items
    (2, 64, 256, 320, 320, 32, "both"),   # the SDXL-2048 conv (128x160 tiles)
    (1, 40, 300, 96, 128, 16, "none"),    # Cin % 64 != 0: 32-wide slices
    (1, 256, 1024, 128, 128, 32, "both"), # a VAE band: 2048 tile rows in one batch item
])
def test_conv_gn_sums(B, h, W, Cin, Cout, G, halos):
    say("conv+gn sums", B, h, W, Cin, Cout, G, halos)
    x = R(1, "cgs.x", (B, h, W, Cin), "bf16")
    w = R(0, "cgs.w", (Cout, 3, 3, Cin), "bf16", (9 * Cin) ** -0.5)
    b = R(3, "cgs.b", (Cout,), "f32", 0.1)
    ht = dev(R(2, "cgs.ht", (B, W, Cin), "bf16"), "bf16") if halos in ("both", "top") else None
    hb = dev(R(2, "cgs.hb", (B, W, Cin), "bf16"), "bf16") if halos in ("both", "bottom") else None
    gx, gw, gb = dev(x, "bf16"), dev(w, "bf16"), dev_f32(b)
    y1 = ops.dp_conv3x3_stale_halo(gx, ht, hb, gw, gb)
    y2, sums = ops.dp_conv3x3_stale_halo_gn_sums(gx, ht, hb, gw, gb, G)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    yh = host(y2).reshape(B, h * W, Cout)
    check_sums(host(sums), yh, G)
    s2 = ops.dp_groupnorm_sums(y2.view(B, h * W, Cout), G)
    assert torch.allclose(sums, s2, rtol=1e-5, atol=1e-3)


@pytest.mark.parametrize("dt,B,T,C,G,N,silu", [("bf16", 2, 7200, 640, 32, 8, False), ("bf16", 1, 5000, 128, 32, 4, True),
                                               ("f32", 2, 300, 64, 8, 3, True)])
def test_groupnorm_apply_equals_stale_stats(dt, B, T, C, G, N, silu):
    x = dev(R(1, "gna.x", (B, T, C), dt), dt)
    st = dev_f32(np.abs(R(2, "gna.st", (N, B, G, 2), "f32")) * T * C / G)
    gm, bt = dev_f32(R(3, "gna.g", (C,), "f32", 0.1) + 1.0), dev_f32(R(3, "gna.b", (C,), "f32", 0.1))
    local = ops.dp_groupnorm_sums(x, G)
    y1 = ops.dp_groupnorm_apply(x, local, st, 1, N * T, gm, bt, 1e-5, silu, G)
    y2 = ops.dp_groupnorm_stale_stats(x, st, 1, N * T, gm, bt, 1e-5, silu, G)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_workspaces_reused_across_calls_and_shapes():
    """One workspace per call kind, used by a run of calls whose tile counts
    and batch sizes change from call to call.  The GroupNorm's ticket
    counters must come back to zero after every call, so each call folds its
    own sums exactly once; the conv's workspace holds only partials its own
    call writes.  Sums against the oracle each time, outputs identical to a
    call on a fresh workspace."""
    gn_shapes = [(2, 7200, 640, 32), (1, 17, 64, 8), (3, 5000, 128, 32), (2, 40000, 320, 32), (1, 1, 64, 32),
                 (2, 7200, 640, 32)]
    need = max(ops.dp_groupnorm_stale_stats_workspace(B, T, C, G) for B, T, C, G in gn_shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (B, T, C, G) in enumerate(gn_shapes * 2):
        say("gn workspace reuse", i, B, T, C, G)
        x = R(40 + i, "wsr.x", (B, T, C), "bf16", 1.3)
        gx = dev(x, "bf16")
        s = ops.dp_groupnorm_sums(gx, G, ws=ws)
        fresh = torch.empty_like(s)
        y = ops.dp_groupnorm_stale_stats(gx, None, 0, T, None, None, 1e-5, i % 2 == 1, G, fresh_sums_out=fresh, ws=ws)
        y_ref = ops.dp_groupnorm_stale_stats(gx, None, 0, T, None, None, 1e-5, i % 2 == 1, G)
        torch.cuda.synchronize()
        check_sums(host(s), x, G)
        assert torch.equal(fresh, s) and torch.equal(y, y_ref)
    conv_shapes = [(2, 30, 240, 640, 640, 32), (3, 7, 50, 64, 64, 8), (2, 13, 100, 64, 160, 32), (1, 40, 300, 96, 128, 16),
                   (1, 256, 1024, 128, 128, 32)]
    need = max(ops.dp_conv3x3_gn_sums_workspace(B, h, W, Co) for B, h, W, Ci, Co, G in conv_shapes)
    # the conv's workspace starts as NaN bytes: every slot its fold reads is
    # written by the same call
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for i, (B, h, W, Cin, Cout, G) in enumerate(conv_shapes * 2):
        say("conv sums workspace reuse", i, B, h, W, Cin, Cout, G)
        x = dev(R(60 + i, "wsr.cx", (B, h, W, Cin), "bf16"), "bf16")
        w = dev(R(0, "wsr.cw", (Cout, 3, 3, Cin), "bf16", (9 * Cin) ** -0.5), "bf16")
        y, sums = ops.dp_conv3x3_stale_halo_gn_sums(x, None, None, w, None, G, ws=ws)
        y_ref, sums_ref = ops.dp_conv3x3_stale_halo_gn_sums(x, None, None, w, None, G)
        torch.cuda.synchronize()
        check_sums(host(sums), host(y).reshape(B, h * W, Cout), G)
        assert torch.equal(y, y_ref) and torch.equal(sums, sums_ref)
