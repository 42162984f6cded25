"""Row-sharded VAE decoder resnet (DistVAE row mode) on the GPU.

- dp_groupnorm_sums against the oracle's group sums, and bit-identical to the
  fresh sums dp_groupnorm_stale_stats reports;
- the small fp32 resnet, sharded over 4 bands, against the oracle's unsharded
  resnet (fp32 tolerance);
- at the KL decoder's 1024^2 levels and the 2048^2 output's full-resolution
  level in bf16 (forward() takes the second GroupNorm's sums from the first
  conv's epilogue): the sharded output agrees with
  the unsharded output computed by the same kernels on the GPU ("Benchmarking
  DistVAE", "Output and exit status": row-sharded agreement is enforced), and
  sampled rows of each layer agree with the oracle computed from the GPU's own
  input to that layer.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from displaced_patch_diffusion_amd import ops, synth
from displaced_patch_diffusion_amd.vae_rows import RowShardedResnet
from tests.util import assert_close, dev, dev_f32, gpu_ok, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_weights(inp, dt):
    w = {}
    for i in range(2):
        w[f"w{i}"] = dev(inp[f"w{i}"], dt)
        for k in ("b", "gamma", "beta"):
            w[f"{k}{i}"] = dev_f32(inp[f"{k}{i}"])
    return w


@pytest.mark.parametrize("dt,B,T,C,G", [("bf16", 2, 7200, 640, 32), ("bf16", 1, 1000, 128, 32),
                                        ("f32", 2, 333, 64, 8), ("bf16", 3, 17, 2048, 32)])
def test_groupnorm_sums(dt, B, T, C, G):
    say("gn sums", dt, B, T, C, G)
    x = synth.random_tensor(1, "gns.x", (B, T, C), dt, 1.5)
    gx = dev(x, dt)
    s = ops.dp_groupnorm_sums(gx, G)
    ref = oracle.group_sums(x, G)
    xa = np.abs(np.asarray(x, np.float64)).reshape(B, T, G, C // G).sum(axis=(1, 3))
    g = host(s)
    assert np.all(np.abs(g[..., 0] - ref[..., 0]) <= 2e-5 * xa + 1e-6)
    assert np.all(np.abs(g[..., 1] - ref[..., 1]) <= 2e-5 * ref[..., 1] + 1e-6)
    fresh = torch.empty_like(s)
    ops.dp_groupnorm_stale_stats(gx, None, 0, T, None, None, 1e-5, False, G, fresh_sums_out=fresh)
    assert torch.equal(fresh, s)


def test_small_fp32_sharded_matches_oracle_unsharded():
    v = synth.VAE_LEVELS["vae_small_fp32"]
    inp = synth.vae_inputs(v)
    net = RowShardedResnet(v.H, v.W, v.C, v.N, gpu_weights(inp, "f32"), v.G, v.eps)
    got = host(net.forward(dev(inp["x"], "f32")))
    x = np.asarray(inp["x"], np.float64)
    B, H, W, C = x.shape
    for i in range(2):
        y, _ = oracle.groupnorm_stale(x.reshape(B, H * W, C), np.zeros((1, B, v.G, 2)), 0, H * W,
                                      inp[f"gamma{i}"], inp[f"beta{i}"], v.eps, True, v.G)
        x = oracle.conv3x3_halo(y.reshape(B, H, W, C), None, None, inp[f"w{i}"], inp[f"b{i}"])
    assert_close(got, x, "f32", "sharded resnet vs unsharded oracle")


def _rows(t, rows):
    """Host float64 copy of image rows `rows` (clipped to the image) of a
    device tensor [B, H, W, C], as a dict row -> [B, W, C]."""
    H = t.shape[1]
    keep = sorted({r for r in rows if 0 <= r < H})
    got = host(t[:, keep])
    return {r: got[:, i] for i, r in enumerate(keep)}


def _layer_check(v, x_in, y_gpu, z_gpu, inp, i, rows, dt):
    """Sampled rows of layer i: the oracle's GroupNorm+SiLU of the device's
    layer input x_in (whole-image statistics from all of x_in) and the oracle's
    conv of the device's own normalised rows y_gpu.  Tensors are [B, H, W, C]
    on the device; only the rows needed are copied to the host."""
    B, H, W, C = x_in.shape
    full = np.zeros((B, v.G, 2))
    step = max(1, (1 << 26) // (B * W * C))  # group sums over the image in slabs of rows
    for r0 in range(0, H, step):
        full += oracle.group_sums(host(x_in[:, r0:r0 + step]).reshape(B, -1, C), v.G)
    xr_all = _rows(x_in, rows)
    yr_all = _rows(y_gpu, [r + d for r in rows for d in (-1, 0, 1)])
    zr_all = _rows(z_gpu, rows)
    for r in rows:
        xr = xr_all[r]
        rest = full - oracle.group_sums(xr, v.G)
        yr, _ = oracle.groupnorm_stale(xr, np.stack([np.zeros_like(rest), rest]), 0, H * W,
                                       inp[f"gamma{i}"], inp[f"beta{i}"], v.eps, True, v.G)
        assert_close(yr_all[r], yr.reshape(B, W, C), dt, f"gn layer {i} row {r}")
        top = yr_all[r - 1] if r > 0 else None
        bot = yr_all[r + 1] if r + 1 < H else None
        zr = oracle.conv3x3_halo(yr_all[r][:, None], top, bot, inp[f"w{i}"], inp[f"b{i}"])
        assert_close(zr_all[r], zr[:, 0], dt, f"conv layer {i} row {r}")


@pytest.mark.parametrize("name", ["vae_kl1024_l1024_c128", "vae_kl1024_l512_c256", "vae_kl2048_l2048_c128"])
def test_rows_agree_with_unsharded_and_oracle(name):
    """Sharded vs unsharded on the GPU (the agreement the DistVAE bench
    enforces), then every layer's rows at the band seams, both image edges and
    one interior row against the oracle."""
    v = synth.VAE_LEVELS[name]
    say("vae rows", name)
    inp = synth.vae_inputs(v)
    wts = gpu_weights(inp, v.dtype)
    x = dev(inp["x"], v.dtype)
    del inp["x"]
    sharded = RowShardedResnet(v.H, v.W, v.C, v.N, wts, v.G, v.eps)
    whole = RowShardedResnet(v.H, v.W, v.C, 1, wts, v.G, v.eps)
    a, b = sharded.forward(x), whole.forward(x)
    torch.cuda.synchronize()
    diff = (a.float() - b.float()).abs().max().item()
    say(f"  max |sharded - unsharded| = {diff:.3g}")
    assert diff <= 2e-2
    del b
    # layer by layer, sampled rows at band seams, image edges and inside a band
    H = v.H
    seams = sorted({0, H - 1} | {e for a0, b0 in sharded.bands for e in (a0, b0 - 1)} | {H // 3})
    xs = [x[:, a0:b0].contiguous() for a0, b0 in sharded.bands]
    x_in = x
    for i in range(2):
        ys = sharded._gn(xs, i)
        zs = sharded._conv(ys, i)
        y_full, z_full = torch.cat(ys, 1), torch.cat(zs, 1)
        del ys
        _layer_check(v, x_in, y_full, z_full, inp, i, seams, v.dtype)
        xs, x_in = zs, z_full
        del y_full
    # forward() takes the second GroupNorm's sums from the first conv's
    # epilogue; the layers above formed them in a pass of their own
    diff = (a.float() - x_in.float()).abs().max().item()
    say(f"  max |forward - layer by layer| = {diff:.3g}")
    assert diff <= 2e-2
