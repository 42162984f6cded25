"""Full-size rank shares, run exactly as the benchmark runs them, checked stage
by stage against the oracle.

The share is built by bench.make_share (same tensors, op list and launch
configuration as the timed steps); only its stale state comes from the seeded
generator (synth.drawn_stale_state, with the stale group sums formed by the
oracle), so that no oracle input depends on the device.  After one step every
stage's stored output is compared with the oracle evaluated on that stage's
stored device input (DistriFusion summary, "How It Works": each share is the
plain layer computation on the rank's rows over spliced stale state):

  single-level:  Q, K and V rows of the fused projection (and the untouched
                 stale rows of the buffers, bit for bit) -> attention (one
                 query row in every 128-query block, every head and batch
                 item, under the planner's schedule and each forced one) ->
                 output projection -> conv with the stale halos (sampled
                 pixels, both band edges) -> GroupNorm with the stale sums
                 (every output) and the fresh sums;
  two-level:     GN+SiLU -> conv -> GN+SiLU -> conv at the conv level, and
                 Q/K/V -> attention -> output projection at the attention
                 level.

Both GroupNorm paths the benchmark offers (sums in a pass of their own, or in
the conv epilogue) and the unfused Q/K/V + splice are run on the same inputs.
test_share_end_to_end compares the step's final output with the oracle's
float64 chain from the step's original inputs (no device intermediate).
"""
from __future__ import annotations

import contextlib
import os
import sys

import numpy as np
import pytest
import torch

import bench
import oracle
from displaced_patch_diffusion_amd import ops, synth
from tests.util import BF16_ATOL, assert_close, gpu_ok, host, max_violation

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]

CHAIN_WORKLOADS = [n for n in synth.WORKLOAD_ORDER if synth.WORKLOADS[n].dtype == "bf16"]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@contextlib.contextmanager
def attn_schedule(name):
    old = os.environ.get("DP_ATTN_SCHEDULE")
    if name is None:
        os.environ.pop("DP_ATTN_SCHEDULE", None)
    else:
        os.environ["DP_ATTN_SCHEDULE"] = name
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("DP_ATTN_SCHEDULE", None)
        else:
            os.environ["DP_ATTN_SCHEDULE"] = old


def block_rows(Tq: int, salt: int = 0) -> np.ndarray:
    """One query row in every 128-query block (its position inside the block
    varies from block to block), plus the last row."""
    rows = {Tq - 1}
    for b0 in range(0, Tq, 128):
        n = min(128, Tq - b0)
        rows.add(b0 + ((b0 // 128) * 53 + 17 + salt) % n)
    return np.array(sorted(rows))


def sample_pixels(h: int, W: int, seed: int):
    """Band rows 0, 1, h/2, h-2, h-1 (both halo rows and the interior) x
    columns 0, 1, W-2, W-1 and 8 random ones."""
    rng = np.random.default_rng(seed)
    rows = sorted({r for r in (0, 1, h // 2, h - 2, h - 1) if 0 <= r < h})
    cols = sorted({c for c in (0, 1, W - 2, W - 1) if 0 <= c < W} | set(rng.choice(W, min(W, 8), replace=False).tolist()))
    return rows, cols


def conv_pixels(x_img, ht, hb, w, b, rows, cols):
    """Oracle conv outputs at (row, col) pixels of a band: each from its
    3-column strip, so the strip's zero padding is the image's.  Returns
    [B, len(rows), len(cols), Cout]."""
    B, h, W, _ = x_img.shape
    out = np.empty((B, len(rows), len(cols), w.shape[0]))
    for a, i in enumerate(rows):
        top = x_img[:, i - 1] if i > 0 else ht
        bot = x_img[:, i + 1] if i < h - 1 else hb
        for c_idx, c in enumerate(cols):
            c0, c1 = max(c - 1, 0), min(c + 2, W)
            strip = oracle.conv3x3_halo(x_img[:, i:i + 1, c0:c1], None if top is None else top[:, c0:c1],
                                        None if bot is None else bot[:, c0:c1], w, b)
            out[:, a, c_idx] = strip[:, 0, c - c0]
    return out


def stale_sums_of(remote, G):
    """The other patches' stale group sums: the oracle's sums of the drawn
    remote activations, stored as float32 as the previous step would."""
    return np.stack([oracle.group_sums(r, G) for r in remote]).astype(np.float32)


def drawn_state(w):
    st = synth.drawn_stale_state(w)
    for i in range(2 if w.two_level else 1):
        st[f"sums{i}"] = stale_sums_of(st.pop(f"remote{i}"), w.G)
    return st


def run_step(share):
    for _, fn in share.ops_:
        fn()
    torch.cuda.synchronize()


def check_sums(gpu_sums, x, G, what):
    """Fresh sums: float32 accumulation, bound 1e-5 * sum |x| (resp. sum x^2)."""
    B, T, C = x.shape
    ref = oracle.group_sums(x, G)
    absx = np.abs(x).reshape(B, T, G, C // G).sum((1, 3))
    g = host(gpu_sums)
    assert (np.abs(g[..., 0] - ref[..., 0]) <= 1e-5 * absx + 1e-6).all(), what
    assert (np.abs(g[..., 1] - ref[..., 1]) <= 1e-5 * ref[..., 1] + 1e-6).all(), what


class Errs:
    """Largest error per stage, printed for the record."""

    def __init__(self, name):
        self.name, self.e = name, {}

    def check(self, gpu, ref, what):
        v = max_violation(gpu, ref, "bf16")
        self.e[what] = max(self.e.get(what, 0.0), v * BF16_ATOL)
        assert v <= 1.0, f"{self.name} {what}: bf16 tolerance exceeded by factor {v:.3g}"

    def report(self):
        say(f"  {self.name} max |err| per stage: " + ", ".join(f"{k} {v:.2e}" for k, v in self.e.items()))


def check_attention_level(w, share, k_stale, v_stale, errs):
    """Q/K/V rows, untouched stale rows, attention on one row per query block
    (planner's pick and each forced schedule), output projection."""
    B, Tq, T_kv, t0 = w.B, w.Tq, w.T_kv, share.t0
    a0, a1 = oracle.partition_rows(w.attn_H, w.N, w.rank)
    assert (t0, Tq) == (a0 * w.attn_W, (a1 - a0) * w.attn_W)
    rows = block_rows(Tq)
    x = host(share.x_loc)
    wq, wk, wv, wo = (host(t) for t in (share.wq, share.wk, share.wv, share.wo))
    q = host(share.q)
    errs.check(q[:, rows], oracle.linear(x[:, rows], wq), "q")
    kb, vb = host(share.k_buf), host(share.v_buf)
    errs.check(kb[:, t0 + rows], oracle.linear(x[:, rows], wk), "k rows")
    errs.check(vb[:, t0 + rows], oracle.linear(x[:, rows], wv), "v rows")
    bits = lambda t: t.view(torch.int16)
    for buf, old in ((share.k_buf, k_stale), (share.v_buf, v_stale)):
        assert torch.equal(bits(buf[:, :t0]), bits(old[:, :t0]))
        assert torch.equal(bits(buf[:, t0 + Tq:]), bits(old[:, t0 + Tq:]))
    ref_o = oracle.attention(q[:, rows], kb, vb, w.heads)
    errs.check(host(share.o)[:, rows], ref_o, "attention")
    for sched in ("split", "balanced"):
        with attn_schedule(sched):
            o2 = ops.dp_attn_stale_kv(share.q, share.k_buf, share.v_buf, w.heads)
        errs.check(host(o2)[:, rows], ref_o, f"attention ({sched})")
        del o2
    errs.check(host(share.y)[:, rows], oracle.linear(host(share.o)[:, rows], wo), "out proj")


def check_conv(w, share, i, x_dev, z_dev, errs, tag):
    B, h, Wd, C = w.B, w.conv_h, w.conv_W, w.conv_C
    cv = share.convs[i]
    x_img = host(x_dev).reshape(B, h, Wd, C)
    ht = None if cv["ht"] is None else host(cv["ht"])
    hb = None if cv["hb"] is None else host(cv["hb"])
    rows, cols = sample_pixels(h, Wd, 31 + i)
    ref = conv_pixels(x_img, ht, hb, host(cv["w"]), host(cv["b"]), rows, cols)
    z = host(z_dev).reshape(B, h, Wd, C)
    errs.check(z[:, rows][:, :, cols], ref, f"conv{i}{tag}")


def check_gn(w, share, i, x_dev, y_dev, errs, tag):
    g = share.gns[i]
    x = host(x_dev)
    ref, _ = oracle.groupnorm_stale(x, host(g["stale"]), w.rank, w.conv_H * w.conv_W, host(g["gamma"]),
                                    host(g["beta"]), w.eps, w.two_level, w.G)
    errs.check(host(y_dev), ref, f"groupnorm{i}{tag}")


def check_conv_level(w, share, errs, tag):
    if w.two_level:
        x = share.conv_in_loc
        for i in range(2):
            check_gn(w, share, i, x, share.gc[i], errs, tag)
            check_conv(w, share, i, share.gc[i], share.zc[i], errs, tag)
            x = share.zc[i]
        # the fresh sums each GroupNorm formed (conv epilogue: the first conv's
        # output feeds the second GroupNorm)
        check_sums(share.fresh[0], host(share.conv_in_loc), w.G, "fresh sums 0")
        check_sums(share.fresh[1], host(share.zc[0]), w.G, "fresh sums 1")
    else:
        check_conv(w, share, 0, share.y, share.zc[0], errs, tag)
        check_gn(w, share, 0, share.zc[0], share.gc[0], errs, tag)
        check_sums(share.fresh[0], host(share.zc[0]), w.G, "fresh sums")


@pytest.mark.parametrize("name", CHAIN_WORKLOADS)
def test_share_step_stagewise(name):
    w = synth.WORKLOADS[name]
    say("chain stage-wise", name)
    share = bench.Share(w, torch, ops, synth, stale=drawn_state(w))
    share.fused_qkv = bench.DEFAULT_QKV == "fused"
    share.gn_sums_in_conv = bench.DEFAULT_GN_SUMS == "conv"
    share.prepare()
    k_stale, v_stale = share.k_buf.clone(), share.v_buf.clone()
    errs = Errs(name)
    run_step(share)
    check_attention_level(w, share, k_stale, v_stale, errs)
    check_conv_level(w, share, errs, "")
    # the other GroupNorm path of the benchmark on the same inputs
    share.gn_sums_in_conv = not share.gn_sums_in_conv
    share.prepare()
    run_step(share)
    check_conv_level(w, share, errs, " (other gn path)")
    # unfused projections + splice: the same buffers and q, bit for bit
    q1, k1, v1 = share.q.clone(), share.k_buf.clone(), share.v_buf.clone()
    share.k_buf.copy_(k_stale)
    share.v_buf.copy_(v_stale)
    share.fused_qkv = not share.fused_qkv
    share.prepare()
    run_step(share)
    assert torch.equal(q1, share.q) and torch.equal(k1, share.k_buf) and torch.equal(v1, share.v_buf)
    errs.report()


# ----------------------------------------------------------- end to end
def e2e_attention_block(inputs, heads, toks):
    """The oracle's float64 attention block at band tokens `toks`, from the
    step's original inputs: the fresh K/V of the whole band spliced into the
    drawn stale buffers."""
    x, wq, wk, wv, wo, kb, vb, t0 = inputs
    k_s, v_s = oracle.kv_buffer_splice(kb, vb, oracle.linear(x, wk), oracle.linear(x, wv), t0)
    o = oracle.attention(oracle.linear(x[:, toks], wq), k_s, v_s, heads)
    return oracle.linear(o, wo)


@pytest.mark.parametrize("name", CHAIN_WORKLOADS)
def test_share_end_to_end(name):
    """The step's final output against the oracle's float64 chain from the
    step's original inputs (no device intermediate).  The single-level shares
    at SDXL-1024^2 and the two-level share's conv level run the whole chain in
    the oracle; at SDXL-3840^2 the oracle evaluates the attention block on the
    query rows feeding sampled conv pixels, and the GroupNorm statistics of the
    whole band (which would need the band's full attention, 2.1 TFLOP in
    float64) are the oracle's sums of the device's conv output.  The errors are
    printed and held to the bf16 tolerance."""
    w = synth.WORKLOADS[name]
    say("chain end to end", name)
    st = drawn_state(w)
    share = bench.Share(w, torch, ops, synth, stale=st)
    share.fused_qkv = bench.DEFAULT_QKV == "fused"
    share.gn_sums_in_conv = bench.DEFAULT_GN_SUMS == "conv"
    share.prepare()
    run_step(share)
    B, Wd, C = w.B, w.attn_W, w.attn_C
    a = synth.attention_block_inputs(w, with_noise=False)
    a0, a1 = oracle.partition_rows(w.attn_H, w.N, w.rank)
    t0 = a0 * Wd
    x = a["x_full"].reshape(B, -1, C)[:, t0:a1 * Wd].astype(np.float64)
    kb, vb = st["k_buf"].astype(np.float64), st["v_buf"].astype(np.float64)
    inputs = (x, a["wq"], a["wk"], a["wv"], a["wo"], kb, vb, t0)
    err = {}
    h = a1 - a0
    if w.two_level:
        # attention level: the block's output rows, one per query block
        rows = block_rows(w.Tq)
        ref_y = e2e_attention_block(inputs, w.heads, rows)
        err["attention block"] = float(np.abs(host(share.y)[:, rows] - ref_y).max())
        # conv level: the whole chain GN+SiLU -> conv -> GN+SiLU -> conv
        c0, c1 = oracle.partition_rows(w.conv_H, w.N, w.rank)
        Hc, Wc, Cc, hc = w.conv_H, w.conv_W, w.conv_C, c1 - c0
        xc = synth.conv_level_input(w).reshape(B, Hc * Wc, Cc)[:, c0 * Wc:c1 * Wc].astype(np.float64)
        for i in range(2):
            cv, gn = synth.conv_inputs(w, i), synth.groupnorm_inputs(w, i)
            g, _ = oracle.groupnorm_stale(xc, st[f"sums{i}"], w.rank, Hc * Wc, gn["gamma"], gn["beta"],
                                          w.eps, True, w.G)
            xc = oracle.conv3x3_halo(g.reshape(B, hc, Wc, Cc), st[f"halo_top{i}"], st[f"halo_bot{i}"],
                                     cv["w"], cv["bias"]).reshape(B, hc * Wc, Cc)
        err["conv level"] = float(np.abs(host(share.zc[1]) - xc).max())
    elif w.T_kv <= 4096:
        cv, gn = synth.conv_inputs(w), synth.groupnorm_inputs(w)
        ref = oracle.rank_share_step(x, a["wq"], a["wk"], a["wv"], a["wo"], kb, vb, t0, w.heads, Wd,
                                     st["halo_top0"], st["halo_bot0"], cv["w"], cv["bias"], st["sums0"],
                                     w.rank, w.T_kv, gn["gamma"], gn["beta"], w.eps, w.G)
        err["attention block"] = float(np.abs(host(share.y) - ref["attn_out"]).max())
        err["conv"] = float(np.abs(host(share.zc[0]) - ref["conv_out"]).max())
        err["step output"] = float(np.abs(host(share.gc[0]) - ref["out"]).max())
    else:
        # sampled conv pixels: the attention block on the tokens feeding them
        cv, gn = synth.conv_inputs(w), synth.groupnorm_inputs(w)
        prow, pcol = sample_pixels(h, Wd, 77)
        need = sorted({(r, c) for i in prow for j in pcol for r in (i - 1, i, i + 1) for c in (j - 1, j, j + 1)
                       if 0 <= r < h and 0 <= c < Wd})
        toks = np.array([r * Wd + c for r, c in need])
        y_need = e2e_attention_block(inputs, w.heads, toks)
        err["attention block"] = float(np.abs(host(share.y)[:, toks] - y_need).max())
        y_img = np.zeros((B, h, Wd, C))
        for n, (r, c) in enumerate(need):
            y_img[:, r, c] = y_need[:, n]
        z_ref = conv_pixels(y_img, st["halo_top0"], st["halo_bot0"], cv["w"], cv["bias"], prow, pcol)
        z_gpu = host(share.zc[0]).reshape(B, h, Wd, C)
        err["conv"] = float(np.abs(z_gpu[:, prow][:, :, pcol] - z_ref).max())
        # GroupNorm of the sampled pixels with the band's statistics taken from
        # the oracle's sums of the device's conv output: an extra stale entry
        # carries (band sums - sums of the sampled pixels)
        pix = z_ref.reshape(B, -1, C)
        extra = oracle.group_sums(host(share.zc[0]), w.G) - oracle.group_sums(pix, w.G)
        stale2 = np.concatenate([st["sums0"].astype(np.float64), extra[None]])
        yg, _ = oracle.groupnorm_stale(pix, stale2, w.rank, w.T_kv, gn["gamma"], gn["beta"], w.eps, False,
                                       w.G)
        got = host(share.gc[0]).reshape(B, h, Wd, C)[:, prow][:, :, pcol].reshape(B, -1, C)
        err["step output (band statistics from the device's conv output)"] = float(np.abs(got - yg).max())
    say(f"  {name} end-to-end max |err|: " + ", ".join(f"{k} {v:.3e}" for k, v in err.items()))
    for k, v in err.items():
        assert v <= E2E_ATOL, f"{name} end to end, {k}: {v:.3e} > {E2E_ATOL}"


# The bf16 tolerance holds end to end as well (largest errors measured on
# MI355X: 1.4e-2 and 1.5e-2 at the two SDXL-1024^2 shares, from q stored in
# bf16 with |q| in [4, 8) and the GroupNorm output's own rounding).
E2E_ATOL = BF16_ATOL
