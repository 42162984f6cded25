#!/usr/bin/env python3
"""Benchmark of one rank's share of a displaced-patch diffusion step on one MI355X.

One step = every hot-path op of the share, in order, through libdp:
  single-level workloads: Q/K/V projections of the local rows with K/V
      written into the full-image buffers (one launch by default; --qkv
      separate runs three projections and then the K/V buffer splice) ->
      attention over the full-image buffer -> output projection ->
      conv3x3 with stale halo rows -> GroupNorm with stale remote sums;
  two-level workload: GN+SiLU -> conv -> GN+SiLU -> conv at the conv level, and
      projections -> splice -> attention -> output projection at the
      attention level.
Inputs are synthetic (seeded) and resident in HBM before timing.  The stale
state (remote K/V rows, halo rows, remote GroupNorm sums) is the previous
step's full-image result plus N(0, 0.05^2) noise, computed on the GPU before
timing.

Prints one JSON line.  value = algorithmic dense FLOPs of the step (attention
+ projections + convs) / measured step time, in TFLOP/s.  The K timed steps
carry HIP events only around the attention call (its average duration gives
roofline.achieved); the per-op breakdown under "kernels" times each op
enqueued K times back to back (every op is idempotent on its inputs), since an
event between ops adds queue time.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
DEFAULT_WORKLOAD = "sdxl3840_l240_c640"
METRIC = "rank-share step TFLOP/s (attn+conv) & GroupNorm GB/s; % of MI355X roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- GPU state
class Share:
    """Device tensors of one rank's share plus its stale state.

    By default the stale state is the previous step's full-image result plus
    N(0, 0.05^2) noise, computed here on the GPU.  `stale` instead hands it in
    as host arrays (the parity tests draw it from the seeded generator): keys
    k_buf, v_buf [B, T_kv, C]; halo_top{i}, halo_bot{i} [B, W, C] or None for
    conv i; sums{i} [N, B, G, 2] float32 for GroupNorm i.  The ops and their
    launch configuration are the same either way."""

    fused_qkv = True
    gn_sums_in_conv = False

    def __init__(self, w, torch, ops, synth, stale=None):
        self.w, self.torch, self.ops = w, torch, ops
        self.dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(self.dt)
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
        opt = lambda a, fn: None if a is None else fn(a)
        noise = lambda name, shape: f32(synth.stale_noise(w, name, shape))
        B = w.B
        # ---------------- attention level
        a = synth.attention_block_inputs(w, with_noise=stale is None)
        H, Wd, C = w.attn_H, w.attn_W, w.attn_C
        T = H * Wd
        x_full = dev(a["x_full"]).view(B, T, C)
        self.wq, self.wk, self.wv, self.wo = (dev(a[k]) for k in ("wq", "wk", "wv", "wo"))
        r0, r1 = w.attn_rows()
        self.t0 = r0 * Wd
        self.x_loc = x_full[:, r0 * Wd:r1 * Wd].contiguous()
        if stale is None:
            k_full = torch.empty((B, T, C), dtype=self.dt, device="cuda")
            v_full = torch.empty_like(k_full)
            for p in range(w.N):
                a0, a1 = w.attn_rows(p)
                xp = x_full[:, a0 * Wd:a1 * Wd].contiguous()
                k_full[:, a0 * Wd:a1 * Wd] = ops.dp_linear(xp, self.wk)
                v_full[:, a0 * Wd:a1 * Wd] = ops.dp_linear(xp, self.wv)
            # stale buffers: the previous step's full-image K/V plus noise
            self.k_buf = (k_full.float() + f32(a["k_noise"])).to(self.dt)
            self.v_buf = (v_full.float() + f32(a["v_noise"])).to(self.dt)
        else:
            self.k_buf, self.v_buf = dev(stale["k_buf"]), dev(stale["v_buf"])
        Tq = w.Tq
        mk = lambda *s: torch.empty(*s, dtype=self.dt, device="cuda")
        self.q, self.kf, self.vf = mk(B, Tq, C), mk(B, Tq, C), mk(B, Tq, C)
        self.o, self.y = mk(B, Tq, C), mk(B, Tq, C)
        self.attn_ws = None
        n = ops.dp_attn_stale_kv_workspace(B, w.heads, Tq, T, C // w.heads, self.dt)
        if n:
            self.attn_ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        # ---------------- conv / GroupNorm level
        G = w.G
        self.G = G
        hc, Wc, Cc, Hc = w.conv_h, w.conv_W, w.conv_C, w.conv_H
        self.hc, Tc = hc, hc * Wc
        self.convs, self.gns = [], []
        n_conv = 2 if w.two_level else 1
        for i in range(n_conv):
            cv = synth.conv_inputs(w, i)
            self.convs.append({"w": dev(cv["w"]), "b": f32(cv["bias"]), "cv": cv})
            gn = synth.groupnorm_inputs(w, i)
            self.gns.append({"gamma": f32(gn["gamma"]), "beta": f32(gn["beta"])})
        rows_c = [w.conv_rows(p) for p in range(w.N)]
        band = lambda full, p: full[:, rows_c[p][0] * Wc:rows_c[p][1] * Wc]
        self.conv_in_loc = None
        if w.two_level:
            z = dev(synth.conv_level_input(w)).view(B, Hc * Wc, Cc)
            self.conv_in_loc = band(z, w.rank).contiguous()
        if stale is not None:
            for i in range(n_conv):
                self.convs[i]["ht"] = opt(stale[f"halo_top{i}"], dev)
                self.convs[i]["hb"] = opt(stale[f"halo_bot{i}"], dev)
                self.gns[i]["stale"] = f32(stale[f"sums{i}"])
        else:
            self._previous_step(w, synth, x_full, k_full, v_full, band, rows_c, f32, noise)
        self.gn_ws = torch.zeros(ops.dp_groupnorm_stale_stats_workspace(B, Tc, Cc, G),
                                 dtype=torch.uint8, device="cuda")
        self.zc = [mk(B, Tc, Cc) for _ in range(2)]
        self.gc = [mk(B, Tc, Cc) for _ in range(2)]
        self.fresh = [torch.empty((B, G, 2), dtype=torch.float32, device="cuda") for _ in range(2)]
        self.conv_ws = torch.zeros(ops.dp_conv3x3_gn_sums_workspace(B, hc, Wc, Cc), dtype=torch.uint8,
                                   device="cuda")
        torch.cuda.synchronize()

    def _previous_step(self, w, synth, x_full, k_full, v_full, band, rows_c, f32, noise):
        """The previous step with stale == fresh, rebuilt rank by rank with the
        same launch shapes as the timed step; stale state = that + noise."""
        torch, ops = self.torch, self.ops
        B, G = w.B, w.G
        Wd = w.attn_W
        hc, Wc, Cc, Hc = w.conv_h, w.conv_W, w.conv_C, w.conv_H
        Tc = hc * Wc

        def halos(full_img, p, noise_t=None, noise_b=None):
            r0, r1 = rows_c[p]
            top = full_img[:, r0 - 1] if r0 > 0 else None
            bot = full_img[:, r1] if r1 < Hc else None
            if noise_t is not None:
                top = None if top is None else (top.float() + noise_t).to(self.dt)
                bot = None if bot is None else (bot.float() + noise_b).to(self.dt)
            return (None if top is None else top.contiguous(), None if bot is None else bot.contiguous())

        def sums_of(full):
            out = torch.zeros((w.N, B, G, 2), dtype=torch.float32, device="cuda")
            for p in range(w.N):
                ops.dp_groupnorm_sums(band(full, p).contiguous(), G, out=out[p])
            return out

        def full_gn(full, i, silu):
            sums = sums_of(full)
            out = torch.empty_like(full)
            for p in range(w.N):
                y = ops.dp_groupnorm_stale_stats(band(full, p).contiguous(), sums, p, Hc * Wc,
                                                 self.gns[i]["gamma"], self.gns[i]["beta"], w.eps,
                                                 silu, G)
                band(out, p).copy_(y)
            return out

        def full_conv(full, i):
            img = full.view(B, Hc, Wc, Cc)
            out = torch.empty((B, Hc * Wc, Cc), dtype=self.dt, device="cuda")
            for p in range(w.N):
                ht, hb = halos(img, p)
                z = ops.dp_conv3x3_stale_halo(band(full, p).contiguous().view(B, rows_c[p][1] - rows_c[p][0],
                                                                               Wc, Cc),
                                              ht, hb, self.convs[i]["w"], self.convs[i]["b"])
                band(out, p).copy_(z.view(B, -1, Cc))
            return out

        def stale_sums(full, i):
            return sums_of((full.float() + noise(f"gn{i}.stale_noise", tuple(full.shape))).to(self.dt))

        def stale_halos(full, i):
            cv = self.convs[i]["cv"]
            return halos(full.view(B, Hc, Wc, Cc), w.rank, f32(cv["halo_top_noise"]),
                         f32(cv["halo_bot_noise"]))

        if w.two_level:
            z = torch.empty((B, Hc * Wc, Cc), dtype=self.dt, device="cuda")
            z.copy_(torch.from_numpy(np.ascontiguousarray(synth.conv_level_input(w), np.float32))
                    .cuda().to(self.dt).view(B, Hc * Wc, Cc))
            for i in range(2):
                self.gns[i]["stale"] = stale_sums(z, i)
                g_full = full_gn(z, i, True)
                self.convs[i]["ht"], self.convs[i]["hb"] = stale_halos(g_full, i)
                z = full_conv(g_full, i)
        else:
            T = w.T_kv
            y_full = torch.empty((B, T, w.attn_C), dtype=self.dt, device="cuda")
            for p in range(w.N):
                a0, a1 = w.attn_rows(p)
                xp = x_full[:, a0 * Wd:a1 * Wd].contiguous()
                y_full[:, a0 * Wd:a1 * Wd] = ops.dp_linear(
                    ops.dp_attn_stale_kv(ops.dp_linear(xp, self.wq), k_full, v_full, w.heads), self.wo)
            self.convs[0]["ht"], self.convs[0]["hb"] = stale_halos(y_full, 0)
            z = full_conv(y_full, 0)
            self.gns[0]["stale"] = stale_sums(z, 0)

    # the ops of one step, in order, as (name, enqueue function)
    def op_list(self):
        w, ops = self.w, self.ops
        B = w.B
        L = []
        if w.two_level:
            hc, Wc, Cc = self.hc, w.conv_W, w.conv_C
            shp = (B, hc, Wc, Cc)
            x = self.conv_in_loc
            for i in range(2):
                gi, ci = self.gns[i], self.convs[i]
                gin, gout, zout, fr = x, self.gc[i], self.zc[i], self.fresh
                if self.gn_sums_in_conv and i == 1:
                    L.append(("groupnorm", lambda gi=gi, gin=gin, gout=gout, fr=fr: ops.dp_groupnorm_apply(
                        gin, fr[1], gi["stale"], w.rank, w.conv_H * Wc, gi["gamma"], gi["beta"], w.eps, True,
                        self.G, y=gout)))
                else:
                    L.append(("groupnorm", lambda gi=gi, gin=gin, gout=gout, fr=fr[i]: ops.dp_groupnorm_stale_stats(
                        gin, gi["stale"], w.rank, w.conv_H * Wc, gi["gamma"], gi["beta"], w.eps, True, self.G,
                        y=gout, fresh_sums_out=fr, ws=self.gn_ws)))
                if self.gn_sums_in_conv and i == 0:
                    # the conv epilogue also forms the local sums the next GroupNorm needs
                    L.append(("conv", lambda ci=ci, gout=gout, zout=zout: ops.dp_conv3x3_stale_halo_gn_sums(
                        gout.view(shp), ci["ht"], ci["hb"], ci["w"], ci["b"], self.G, y=zout.view(shp),
                        gn_sums=self.fresh[1], ws=self.conv_ws)))
                else:
                    L.append(("conv", lambda ci=ci, gout=gout, zout=zout: ops.dp_conv3x3_stale_halo(
                        gout.view(shp), ci["ht"], ci["hb"], ci["w"], ci["b"], y=zout.view(shp))))
                x = zout
        if self.fused_qkv:
            # one launch: Q/K/V of the local rows, K and V written into the buffers
            L.append(("proj", lambda: ops.dp_qkv_projection_into_buffers(
                self.x_loc, self.wq, self.wk, self.wv, self.k_buf, self.v_buf, self.t0, q=self.q)))
        else:
            def three():
                ops.dp_linear(self.x_loc, self.wq, y=self.q)
                ops.dp_linear(self.x_loc, self.wk, y=self.kf)
                ops.dp_linear(self.x_loc, self.wv, y=self.vf)
            L.append(("proj", three))
            L.append(("splice", lambda: ops.dp_kv_buffer_splice(self.k_buf, self.v_buf, self.kf, self.vf,
                                                                self.t0)))
        L.append(("attn", lambda: ops.dp_attn_stale_kv(self.q, self.k_buf, self.v_buf, w.heads, out=self.o,
                                                        ws=self.attn_ws)))
        L.append(("proj", lambda: ops.dp_linear(self.o, self.wo, y=self.y)))
        if not w.two_level:
            c, g = self.convs[0], self.gns[0]
            shp = (B, self.hc, w.conv_W, w.conv_C)
            if self.gn_sums_in_conv:
                # the conv epilogue forms the GroupNorm's local sums; the GroupNorm is one pass
                L.append(("conv", lambda: ops.dp_conv3x3_stale_halo_gn_sums(
                    self.y.view(shp), c["ht"], c["hb"], c["w"], c["b"], self.G, y=self.zc[0].view(shp),
                    gn_sums=self.fresh[0], ws=self.conv_ws)))
                L.append(("groupnorm", lambda: ops.dp_groupnorm_apply(
                    self.zc[0], self.fresh[0], g["stale"], w.rank, w.conv_H * w.conv_W, g["gamma"], g["beta"],
                    w.eps, False, self.G, y=self.gc[0])))
            else:
                L.append(("conv", lambda: ops.dp_conv3x3_stale_halo(
                    self.y.view(shp), c["ht"], c["hb"], c["w"], c["b"], y=self.zc[0].view(shp))))
                L.append(("groupnorm", lambda: ops.dp_groupnorm_stale_stats(
                    self.zc[0], g["stale"], w.rank, w.conv_H * w.conv_W, g["gamma"], g["beta"], w.eps, False,
                    self.G, y=self.gc[0], fresh_sums_out=self.fresh[0], ws=self.gn_ws)))
        return L

    def gn_moved_bytes(self) -> int:
        """Bytes the step's GroupNorms move: read x and write y, plus one more
        read of x for each GroupNorm that forms its own sums."""
        w = self.w
        one = w.B * w.conv_T * w.conv_C * w.elem_bytes
        if w.two_level:  # the first GroupNorm always forms its own sums
            return 3 * one + (2 if self.gn_sums_in_conv else 3) * one
        return (2 if self.gn_sums_in_conv else 3) * one

    def outputs(self):
        """Tensors the step writes and no op reads before writing (the K/V
        buffers, updated in place, are left out)."""
        n = 2 if self.w.two_level else 1
        return [self.q, self.o, self.y, *self.zc[:n], *self.gc[:n], *self.fresh[:n]]

    # one step; `mark(name)` is called after each op is enqueued
    def step(self, mark):
        for name, fn in self.ops_:
            fn()
            mark(name)

    def prepare(self):
        self.ops_ = self.op_list()


DEFAULT_QKV = "fused"
DEFAULT_GN_SUMS = "conv"


def make_share(w, qkv: str = DEFAULT_QKV, gn_sums: str = DEFAULT_GN_SUMS):
    """The share of workload `w` with its stale state on the GPU, its op list
    prepared exactly as the timed steps run it."""
    import torch

    from displaced_patch_diffusion_amd import ops, synth

    share = Share(w, torch, ops, synth)
    share.fused_qkv = qkv == "fused"
    share.gn_sums_in_conv = gn_sums == "conv"
    share.prepare()
    return share


def back_to_back_us(torch, fn, reps: int) -> float:
    """Average duration of `fn`'s launches, enqueued `reps` times back to back
    between two events behind a GPU spin that lets the host queue them all (no
    host launch latency and no per-call event inside the interval)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(2_000_000)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


# ------------------------------------------------------------ OTIL transmit
def otil_timing(torch, ops, synth, steps: int):
    """OTIL selective transmit at the pages' setting (SDXL 1024^2, 4 ranks,
    --otil_k 32): the fp16 latent band of one rank (32 x 128 pixels, C = 4,
    batch 2) in 8 x 8 blocks (K = 64), k = 32.  One sender step
    (dp_otil_select_pack) and the receiver's copies from the 3 peers
    (dp_otil_unpack), timed with HIP events on the launch stream."""
    B, h, W, C, N, bh, bw, k = 2, 32, 128, 4, 4, 8, 8, 32
    H, K = N * h, (h // bh) * (W // bw)
    seq = synth.otil_latent_sequence(9, B, H, W, C, 2, bh, bw, "f16")
    dv = lambda a: torch.from_numpy(a).cuda().to(torch.float16).contiguous()
    band, last = dv(seq[1][:, h:2 * h]), dv(seq[0][:, h:2 * h])
    vis = torch.ones(K, dtype=torch.uint8, device="cuda")
    copy = dv(seq[0])
    scores = torch.empty(K, dtype=torch.float32, device="cuda")
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    packed = torch.empty((k, B, bh, bw, C), dtype=torch.float16, device="cuda")
    last0 = last.clone()

    # Every select_pack call scores all K blocks and packs k of them, whatever
    # the visited flags and last-sent state left by the call before, so the
    # calls repeat the same work back to back; unpack copies k blocks.
    t_s = back_to_back_us(torch, lambda: ops.dp_otil_select_pack(band, last, vis, bh, bw, k, scores=scores, idx=idx,
                                                                 packed=packed), steps)
    t_u = back_to_back_us(torch, lambda: ops.dp_otil_unpack(copy, packed, idx, 2 * h, h, bh, bw), steps)
    es = 2
    band_b = B * h * W * C * es
    blk_b = k * B * bh * bw * C * es
    send_bytes = 2 * band_b + 3 * blk_b    # score reads x, last_sent; pack reads k blocks, writes packed + last_sent
    unpack_bytes = 2 * blk_b               # per peer: read packed, write the blocks
    return {"workload": "SDXL 1024^2 latent band 32x128, C=4, batch 2, fp16, 8x8 blocks, K=64, k=32, 4 ranks",
            "select_pack_us": round(t_s, 2), "unpack_us_per_peer": round(t_u, 2),
            "select_pack_bytes": send_bytes, "unpack_bytes_per_peer": unpack_bytes,
            "select_pack_GBps": round(send_bytes / t_s / 1e3, 2),
            "bound": "launch latency (the band is 64 KB; at 8 TB/s its bytes take 0.03 us)"}


# ---------------------------------------------------- row-sharded VAE decoder
def vae_rows_timing(torch, ops, synth, name: str, steps: int):
    """One rank's band of a KL-VAE decoder resnet in DistVAE's row mode: group
    sums, GN+SiLU with the other bands' current sums, conv3x3 with fresh halos,
    twice.  The neighbour bands' halos and sums are computed once beforehand;
    only the rank's own calls are timed, each op back to back and the whole
    band step back to back."""
    from displaced_patch_diffusion_amd.vae_rows import RowShardedResnet
    v = synth.VAE_LEVELS[name]
    inp = synth.vae_inputs(v)
    dt = torch.bfloat16 if v.dtype == "bf16" else torch.float32
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(dt)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    wts = {}
    for i in range(2):
        wts[f"w{i}"] = dv(inp[f"w{i}"])
        for k in ("b", "gamma", "beta"):
            wts[f"{k}{i}"] = f32(inp[f"{k}{i}"])
    net = RowShardedResnet(v.H, v.W, v.C, v.N, wts, v.G, v.eps)
    x = dv(inp["x"])
    B, r = v.B, v.rank
    # the state a real run gets from its neighbours: per layer, all bands' sums
    # and the halo rows of the normalised neighbour bands
    xs = [x[:, a:b].contiguous() for a, b in net.bands]
    layer = []
    for i in range(2):
        sums = torch.stack([ops.dp_groupnorm_sums(t.view(B, -1, v.C), v.G) for t in xs])
        ys = net._gn(xs, i)
        layer.append((sums, ys[r - 1][:, -1].contiguous() if r > 0 else None,
                      ys[r + 1][:, 0].contiguous() if r + 1 < v.N else None))
        xs = net._conv(ys, i)
    x0 = x[:, net.bands[r][0]:net.bands[r][1]].contiguous()
    h = x0.shape[1]
    T = h * v.W
    ws = torch.zeros(ops.dp_groupnorm_stale_stats_workspace(B, T, v.C, v.G), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x0)
    z = [torch.empty_like(x0), torch.empty_like(x0)]
    own = torch.empty((B, v.G, 2), dtype=torch.float32, device="cuda")
    own1 = torch.empty_like(own)
    conv_ws = torch.zeros(ops.dp_conv3x3_gn_sums_workspace(B, h, v.W, v.C), dtype=torch.uint8, device="cuda")

    def gn_op(i, xin, local):
        sums = layer[i][0]
        return ("gn", lambda: ops.dp_groupnorm_apply(xin.view(B, T, v.C), local, sums, r, v.H * v.W,
                                                     wts[f"gamma{i}"], wts[f"beta{i}"], v.eps, True, v.G,
                                                     y=y.view(B, T, v.C)))

    _, top0, bot0 = layer[0]
    _, top1, bot1 = layer[1]
    # layer 0: sums pass, GN+SiLU, conv whose epilogue forms the next GroupNorm's
    # sums; layer 1: GN+SiLU in one pass, conv
    band_ops = [("sums", lambda: ops.dp_groupnorm_sums(x0.view(B, T, v.C), v.G, out=own, ws=ws)),
                gn_op(0, x0, own),
                ("conv_gn", lambda: ops.dp_conv3x3_stale_halo_gn_sums(y, top0, bot0, wts["w0"], wts["b0"], v.G,
                                                                      y=z[0], gn_sums=own1, ws=conv_ws)),
                gn_op(1, z[0], own1),
                ("conv", lambda: ops.dp_conv3x3_stale_halo(y, top1, bot1, wts["w1"], wts["b1"], y=z[1]))]

    def band_step():
        for _, fn in band_ops:
            fn()

    for _ in range(3):
        band_step()
    torch.cuda.synchronize()
    # per op: its launches back to back (each op is idempotent on its inputs),
    # averaged over the two layers; the whole band step back to back as well
    acc = {"sums": [], "gn": [], "conv": [], "conv_gn": []}
    for name, fn in band_ops:
        acc[name].append(back_to_back_us(torch, fn, steps))
    med = {k: float(np.mean(a)) for k, a in acc.items()}
    resnet = back_to_back_us(torch, band_step, steps)
    fl, gb = v.conv_flops(), v.gn_bytes()
    gn_total = med["sums"] + 2 * med["gn"]  # both GroupNorms of the resnet
    return {"workload": f"{v.name}: {v.note}; band {h}x{v.W}x{v.C}, batch {B}, rank {r} of {v.N}",
            "conv_us": round(med["conv"], 2), "conv_TFLOPs": round(fl / med["conv"] / 1e6, 1),
            "conv_frac": round(fl / med["conv"] / 1e6 / PEAK_BF16_TFLOPS, 4),
            "conv_with_gn_sums_us": round(med["conv_gn"], 2),
            "groupnorm_sums_us": round(med["sums"], 2), "groupnorm_apply_us": round(med["gn"], 2),
            "groupnorm_GBps": round(2 * gb / gn_total / 1e3, 1),
            "groupnorm_frac": round(2 * gb / gn_total / 1e3 / PEAK_HBM_GBPS, 4),
            "resnet_us": round(resnet, 2),
            "note": "the first conv's epilogue forms the second GroupNorm's sums; groupnorm_* cover both "
                    "GroupNorms (one sums pass, two apply passes)"}


# -------------------------------------------------------------- CPU baseline
def cpu_baseline(w, synth, seconds: float):
    """The oracle, as it stands, on a bounded sample of the same share; each
    op's sample time is scaled up by its own sampled fraction.  The number of
    query rows is chosen from a 4-row probe so that the attention sample takes
    about `seconds` on this host."""
    import oracle

    oracle.build()
    dt = w.dtype
    R = synth.random_tensor
    B, C, Tkv = w.B, w.attn_C, w.T_kv
    t = {}
    k = R(1, "cpu.k", (B, Tkv, C), dt)
    v = R(1, "cpu.v", (B, Tkv, C), dt)
    wl = R(0, "cpu.w", (C, C), dt, C ** -0.5)
    probe = min(4, w.Tq)
    t0 = time.perf_counter()
    oracle.attention(R(1, "cpu.q0", (B, probe, C), dt), k, v, w.heads)
    per_row = (time.perf_counter() - t0) / probe
    rows = int(max(8, min(w.Tq, seconds / max(per_row, 1e-9))))
    q = R(1, "cpu.q", (B, rows, C), dt)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, w.heads)
    t["attn"] = (time.perf_counter() - t0) * w.Tq / rows
    t0 = time.perf_counter()
    for _ in range(4):
        oracle.linear(q, wl)
    t["proj"] = (time.perf_counter() - t0) * w.Tq / rows
    t0 = time.perf_counter()
    oracle.kv_buffer_splice(k[:, :w.Tq], v[:, :w.Tq], q, q, 0)
    t["splice"] = (time.perf_counter() - t0) * w.Tq / rows
    Cc, Wc, hc = w.conv_C, w.conv_W, w.conv_h
    n_conv = 2 if w.two_level else 1
    xr = R(1, "cpu.xc", (B, 1, Wc, Cc), dt)
    hr = R(2, "cpu.hc", (B, Wc, Cc), dt)
    cw = R(0, "cpu.cw", (Cc, 3, 3, Cc), dt, (9 * Cc) ** -0.5)
    t0 = time.perf_counter()
    oracle.conv3x3_halo(xr, hr, hr, cw, None)
    t["conv"] = (time.perf_counter() - t0) * hc * n_conv
    st = np.zeros((w.N, B, w.G, 2))
    t0 = time.perf_counter()
    oracle.groupnorm_stale(xr.reshape(B, Wc, Cc), st, w.rank, w.N * hc * Wc, None, None, w.eps,
                           w.two_level, w.G)
    t["groupnorm"] = (time.perf_counter() - t0) * hc * n_conv
    fl = w.flops()
    total = sum(t.values())
    return {
        "value": sum(fl.values()) / total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count()),
        "kind": "oracle",
        "sample": (f"{rows} of {w.Tq} query rows x {B} batch items against all {Tkv} keys "
                   f"(attention, projections, splice); 1 of {hc} output rows per conv and per "
                   f"GroupNorm; fp64 C oracle, each op's time scaled by its sampled fraction"),
        "step_s_extrapolated": total,
        "per_op_s_extrapolated": {k2: round(v2, 3) for k2, v2 in t.items()},
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


# ----------------------------------------------------------- counter traffic
def _traffic_from_profile(w):
    """L2<->fabric bytes per call of the attention op (its kernels summed)
    from the committed rocprofv3 counter summary of this workload, if that
    summary was taken on the current attention source."""
    from displaced_patch_diffusion_amd import build, rocprof_summary

    rec = rocprof_summary.read_result(os.path.join(ROOT, "profiles", f"counters_{w.name}.txt"))
    if not rec:
        return None
    now = build.source_digest()
    if any(rec.get("sources_sha256", {}).get(f) != now.get(f) for f in ("attention.hip", "dp_internal.h")):
        return None
    a = rec.get("ops", {}).get("attn", {})
    if "read_bytes" not in a or "write_bytes" not in a:
        return None
    return int(a["read_bytes"] + a["write_bytes"])


# ------------------------------------------------------------------ timing
class Flusher:
    """A 1 GiB buffer written before every cold repetition, outside its event
    pair: larger than the eight 4 MB L2s and the 256 MB last-level cache, so a
    cold repetition reads its inputs from HBM."""

    BYTES = 1 << 30

    def __init__(self, torch):
        self.buf = torch.empty(self.BYTES, dtype=torch.uint8, device="cuda")

    def __call__(self):
        self.buf.zero_()


def event_medians_us(torch, fn, reps: int, flush=None) -> float:
    """Median over `reps` repetitions of [flush;] event; fn(); event, in us.
    All pairs are recorded on torch's current stream, where every library
    call launches, and read after one synchronisation."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    fn()
    torch.cuda.synchronize()
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]))


def measure_ops(torch, share, K: int, reps: int, flush):
    """Per op of the step (ops of one name summed): the back-to-back average
    of K launches (hot; the per-op figure the fractions use), and the hot and
    cold (flushed) medians of single launches between an event pair (these
    include an event pair's few microseconds of queue time)."""
    b2b, hot, cold = {}, {}, {}
    for name, fn in share.ops_:
        b2b[name] = b2b.get(name, 0.0) + back_to_back_us(torch, fn, K)
        hot[name] = hot.get(name, 0.0) + event_medians_us(torch, fn, reps)
        if flush is not None:
            cold[name] = cold.get(name, 0.0) + event_medians_us(torch, fn, reps, flush)
    return b2b, hot, cold


def kernel_table(w, b2b, hot, cold, moved=None):
    """Per-op records; `moved` maps an op to the bytes its kernels move when
    that differs from the algorithmic count (a GroupNorm that forms its own
    sums reads x twice)."""
    fl, by = w.flops(), w.bytes()
    peak_mfma = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    kern = {}
    for name, t in b2b.items():
        c = cold.get(name)
        rec = {"us": round(t, 2), "us_hot_median": round(hot[name], 2),
               "us_cold_median": None if c is None else round(c, 2)}
        if name in fl:
            a = fl[name] / t / 1e6
            rec.update({"TFLOP/s": round(a, 1), "frac": round(a / peak_mfma, 4),
                        "frac_cold": None if c is None else round(fl[name] / c / 1e6 / peak_mfma, 4)})
        elif name in by:
            a = by[name] / t / 1e3
            rec.update({"GB/s": round(a, 1), "frac": round(a / PEAK_HBM_GBPS, 4),
                        "frac_cold": None if c is None else round(by[name] / c / 1e3 / PEAK_HBM_GBPS, 4)})
            if moved and name in moved and moved[name] != by[name]:
                rec.update({"moved_bytes": moved[name], "moved_GB/s": round(moved[name] / t / 1e3, 1)})
        kern[name] = rec
    return kern


def splice_timing(torch, ops, share, K: int, reps: int, flush):
    """The K/V buffer splice at the share's shape (the step itself writes K/V
    straight from the projection): fresh rows into both full-image buffers."""
    w = share.w
    fn = lambda: ops.dp_kv_buffer_splice(share.k_buf, share.v_buf, share.kf, share.vf, share.t0)
    t = back_to_back_us(torch, fn, K)
    cold = event_medians_us(torch, fn, reps, flush) if flush is not None else None
    by = w.bytes()["splice"]
    return {"us": round(t, 2), "GB/s": round(by / t / 1e3, 1), "frac": round(by / t / 1e3 / PEAK_HBM_GBPS, 4),
            "us_cold_median": None if cold is None else round(cold, 2),
            "frac_cold": None if cold is None else round(by / cold / 1e3 / PEAK_HBM_GBPS, 4), "bytes": by}


def config_summary(torch, ops, synth, name: str, K: int, reps: int, flush):
    """Another workload's share: per-op numbers and the step's medians."""
    w = synth.WORKLOADS[name]
    # the conv epilogue forms GroupNorm sums in bf16 only
    share = make_share(w, DEFAULT_QKV, DEFAULT_GN_SUMS if w.dtype == "bf16" else "separate")
    for _ in range(3):
        share.step(lambda n: None)
    torch.cuda.synchronize()
    b2b, hot, cold = measure_ops(torch, share, K, reps, flush)
    step = lambda: share.step(lambda n: None)
    step_hot = event_medians_us(torch, step, reps)
    step_cold = event_medians_us(torch, step, reps, flush) if flush is not None else None
    fl = w.flops()
    out = {"workload": w.name, "note": w.note, "dtype": w.dtype,
           "step_us_hot_median": round(step_hot, 2),
           "step_us_cold_median": None if step_cold is None else round(step_cold, 2),
           "TFLOP/s_hot": round(sum(fl.values()) / step_hot / 1e6, 1),
           "kernels": kernel_table(w, b2b, hot, cold, {"groupnorm": share.gn_moved_bytes()})}
    if w.dtype == "bf16":
        out["splice"] = splice_timing(torch, ops, share, K, reps, flush)
    out["graph"] = graph_timing(torch, share, K, reps, flush)
    del share
    torch.cuda.empty_cache()
    return out


def graph_timing(torch, share, K: int, reps: int, flush):
    """The step captured once as a HIP graph (torch.cuda.CUDAGraph) and
    replayed: back-to-back average and hot/cold medians per replay.  Before
    timing, three replays, each after the step's outputs were cleared by eager
    work, must reproduce the eager step's outputs bit for bit."""
    noop = lambda n: None
    try:
        outs = share.outputs()
        share.step(noop)
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            share.step(noop)
        torch.cuda.synchronize()
        match = True
        for _ in range(3):
            for t in outs:
                t.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            match = match and all(torch.equal(a, b) for a, b in zip(outs, ref))
        if not match:
            return {"replays_match_eager": False}
        t = back_to_back_us(torch, g.replay, K)
        hot = event_medians_us(torch, g.replay, reps)
        cold = event_medians_us(torch, g.replay, reps, flush) if flush is not None else None
        del g
        return {"replays_match_eager": True, "step_us": round(t, 2), "step_us_hot_median": round(hot, 2),
                "step_us_cold_median": None if cold is None else round(cold, 2)}
    except Exception as e:  # capture not available: reported, not fatal
        return {"error": f"{type(e).__name__}: {e}"}


# ------------------------------------------------------------ profile runs
def profile_ops(torch, ops, share, reps: int, flush=None):
    """For rocprofv3 runs: each op of the step launched `reps` times in a row,
    in step order, then the K/V splice on the share's buffers (a plain copy of
    known size, the counters' calibration).  A `torch.cuda._sleep` spin kernel
    precedes each op's run and follows the last one, so the dispatch records
    split at the spins and every segment belongs to one op.  With `flush`,
    every launch follows a cache flush (a torch fill kernel, which the
    summariser drops).  Returns the segment labels, which the run prints for
    the summariser."""
    labels, fns, seen = [], [], {}
    for name, fn in share.ops_:
        k = seen.get(name, 0)
        seen[name] = k + 1
        if name == "proj":
            lab = ("qkv_proj" if k == 0 else "out_proj")
        else:
            lab = f"{name}{k}" if name in ("conv", "groupnorm") else name
        labels.append(lab)
        fns.append(fn)
    labels.append("splice_copy")
    fns.append(lambda: ops.dp_kv_buffer_splice(share.k_buf, share.v_buf, share.kf, share.vf, share.t0))
    torch.cuda.synchronize()
    for fn in fns:
        torch.cuda._sleep(1000)
        for _ in range(reps):
            if flush is not None:
                flush()
            fn()
        torch.cuda.synchronize()
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    return labels


# ---------------------------------------------------------------- provenance
def provenance(torch):
    """Where the numbers come from: build revision and source digests,
    ROCm/HIP/torch versions, device and its clocks as the SMI tools report
    them after the timed work, host CPU."""
    import subprocess

    from displaced_patch_diffusion_amd import build as b

    out = {}
    try:
        with open(b.BUILD_INFO) as f:
            info = json.load(f)
        out["build_git_rev"] = info.get("git_rev")
        out["hipcc"] = info.get("hipcc")
        out["sources_match_build"] = info.get("sources_sha256") == b.source_digest()
    except (OSError, ValueError):
        out["build_git_rev"] = None
    out["sources_sha256_16"] = {k: v[:16] for k, v in b.source_digest().items()}
    try:
        with open("/opt/rocm/.info/version") as f:
            out["rocm_version"] = f.read().strip()
    except OSError:
        out["rocm_version"] = None
    out["torch"] = torch.__version__
    out["torch_hip"] = getattr(torch.version, "hip", None)
    props = torch.cuda.get_device_properties(0)
    out["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "compute_units": props.multi_processor_count, "hbm_GiB": round(props.total_memory / 2 ** 30, 1)}
    clocks = None
    for cmd in (["rocm-smi", "--showclocks", "--json"], ["amd-smi", "metric", "--clock", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
            if r.returncode == 0 and r.stdout.strip():
                clocks = {"tool": cmd[0], "report": json.loads(r.stdout)}
                break
        except (OSError, subprocess.SubprocessError, ValueError):
            continue
    out["clocks_after_timing"] = clocks
    out["host"] = {"cpu_model": _cpu_model(), "cpus": os.cpu_count()}
    return out


# ---------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=50, help="repetitions behind every hot and cold median")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle's attention sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gn-sums", choices=("conv", "separate"), default=DEFAULT_GN_SUMS,
                    help="conv: the conv epilogue forms the GroupNorm's local sums and the GroupNorm is one "
                         "pass; separate: the GroupNorm forms them in a read pass of its own")
    ap.add_argument("--no-otil", action="store_true", help="skip the OTIL selective-transmit timing")
    ap.add_argument("--no-vae", action="store_true", help="skip the row-sharded VAE decoder timing")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' numbers")
    ap.add_argument("--seed", type=int, default=0,
                    help="another family of seeded input streams (0: the one the tests use)")
    ap.add_argument("--noise", type=float, default=None, help="std of the stale-state noise (default: the workload's)")
    ap.add_argument("--rank", type=int, default=None, help="which rank's share to time (default: the workload's)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cold (cache-flushed) medians")
    ap.add_argument("--profile-ops", type=int, default=0, metavar="R",
                    help="rocprofv3 mode: launch each op of the step R times in step order, spin kernels "
                         "between the ops, print the op labels and exit (no timing)")
    ap.add_argument("--profile-flush", action="store_true",
                    help="with --profile-ops: flush the caches (1 GiB write) before every launch")
    ap.add_argument("--qkv", choices=("fused", "separate"), default=DEFAULT_QKV,
                    help="fused: one launch projects Q/K/V and writes K/V into the buffers; "
                         "separate: three projections then the K/V splice")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one rank's share on ONE GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from displaced_patch_diffusion_amd import ops, synth

    if args.workload not in synth.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; choose from {list(synth.WORKLOADS)}")
    w = synth.WORKLOADS[args.workload]
    if args.rank is not None:
        if not 0 <= args.rank < w.N:
            sys.exit(f"--rank must be in [0, {w.N}) for {w.name}")
        w = w.with_rank(args.rank)
    if args.noise is not None:
        w = w.with_noise(args.noise)
    synth.set_stream_salt(args.seed)
    torch.cuda.set_device(0)
    if w.dtype != "bf16" and args.gn_sums == "conv":
        log("bench: the conv epilogue forms GroupNorm sums in bf16 only; using --gn-sums separate")
        args.gn_sums = "separate"
    log(f"bench: workload {w.name}: building inputs")
    share = make_share(w, args.qkv, args.gn_sums)
    names = []

    def collect(name):
        names.append(name)

    share.step(collect)
    for _ in range(args.warmup):
        share.step(lambda n: None)
    torch.cuda.synchronize()

    if args.profile_ops:
        labels = profile_ops(torch, ops, share, args.profile_ops, Flusher(torch) if args.profile_flush else None)
        print("PROFILE_OPS " + json.dumps({"workload": w.name, "reps": args.profile_ops, "labels": labels,
                                           "flush": bool(args.profile_flush),
                                           "qkv": args.qkv, "gn_sums": args.gn_sums,
                                           "splice_bytes": w.bytes()["splice"]}), flush=True)
        return
    flush = None if args.no_flush else Flusher(torch)
    K, R = args.steps, args.reps
    # Per-op breakdown, before the timed steps: the back-to-back average of K
    # launches of each op (behind a GPU spin that lets the host queue them
    # all, so neither event queue time nor host launch time enters it), and
    # hot and cold medians of single launches.
    log("bench: per-op timings")
    b2b, hot, cold = measure_ops(torch, share, K, R, flush)
    # Timed region: K steps with HIP events only around the attention call (on
    # torch's current stream, where every library call launches); an event
    # between every op costs a few microseconds of queue time each.
    i_attn = names.index("attn")
    att = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        pos = [0]

        def mark_attn(name, pair=att[s], pos=pos):
            if pos[0] == i_attn - 1:
                pair[0].record()
            elif name == "attn":
                pair[1].record()
            pos[0] += 1

        if i_attn == 0:
            att[s][0].record()
        share.step(mark_attn)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"bench: {K} steps in {wall:.4f}s")
    attn_t = sum(a.elapsed_time(b) for a, b in att) * 1e-3 / K
    # the whole step's medians, after the timed region
    step = lambda: share.step(lambda n: None)
    step_hot = event_medians_us(torch, step, R)
    step_cold = event_medians_us(torch, step, R, flush) if flush is not None else None

    fl = w.flops()
    step_s = wall / K
    work = sum(fl.values())
    value = work / step_s / 1e12
    peak_mfma = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    b2b["attn"] = attn_t * 1e6  # the timed steps' own attention time
    kern = kernel_table(w, b2b, hot, cold, {"groupnorm": share.gn_moved_bytes()})
    achieved = fl["attn"] / attn_t / 1e12
    bf = w.dtype == "bf16"
    roofline = {"bound": "mfma" if bf else "alu", "achieved": round(achieved, 2), "peak": peak_mfma,
                "unit": "TFLOP/s", "frac": round(achieved / peak_mfma, 4),
                "traffic": _traffic_from_profile(w), "kernel": "attn_bf16_d64" if bf else f"attn_f32<{w.head_dim}>",
                "work_per_launch": f"{fl['attn'] / 1e9:.2f} GFLOP"}
    splice = splice_timing(torch, ops, share, K, R, flush) if w.dtype == "bf16" else None
    log("bench: the step as a HIP graph")
    graph = graph_timing(torch, share, K, R, flush)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "strong", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "attn_level": f"{w.attn_H}x{w.attn_W}",
                   "C_attn": w.attn_C, "heads": w.heads, "head_dim": w.head_dim,
                   "conv_level": f"{w.conv_H}x{w.conv_W}", "C_conv": w.conv_C, "n_patches": w.N,
                   "rank": w.rank, "Tq": w.Tq, "T_kv": w.T_kv, "qkv": args.qkv, "gn_sums": args.gn_sums,
                   "noise": w.noise, "seed": args.seed,
                   "parallelism": "one rank's share, 1 GPU"},
        "roofline": roofline,
        "kernels": kern,
        "groupnorm_GBps": kern.get("groupnorm", {}).get("GB/s"),
        "splice": splice,
        "graph": graph,
        "step_us_hot_median": round(step_hot, 2),
        "step_us_cold_median": None if step_cold is None else round(step_cold, 2),
        "timing": {"reps": R, "flush_bytes": None if flush is None else Flusher.BYTES,
                   "per_op_us": "average of K back-to-back launches (hot)",
                   "medians": "median of reps single launches between an event pair; cold reps flush "
                              "the caches with a 1 GiB write outside the pair"},
        "flops_counted": {k2: v2 for k2, v2 in fl.items()},
    }
    del share
    torch.cuda.empty_cache()
    if not args.no_configs:
        others = [n for n in synth.WORKLOAD_ORDER if n != w.name]
        out["configs"] = {}
        for n in others:
            log(f"bench: workload {n}")
            out["configs"][n] = config_summary(torch, ops, synth, n, 10, 20, flush)
    if not args.no_otil:
        out["otil"] = otil_timing(torch, ops, synth, 20)
    if not args.no_vae:
        out["vae_rows"] = [vae_rows_timing(torch, ops, synth, n, 10)
                           for n in ("vae_kl1024_l1024_c128", "vae_kl2048_l2048_c128")]
    if not args.no_cpu_baseline:
        log("bench: CPU baseline (oracle on a bounded sample)")
        out["cpu_baseline"] = cpu_baseline(w, synth, args.cpu_seconds)
        out["cpu_baseline"]["gpu_over_cpu"] = round(value / out["cpu_baseline"]["value"], 1)
    out["provenance"] = provenance(torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
