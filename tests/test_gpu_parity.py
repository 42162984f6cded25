"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.  Small cases span several tiles with ragged tails;
full-size cases use the shapes and launch configuration the benchmark times
and check sampled outputs the oracle computes one by one (or every output
where the oracle is cheap).  Tolerances are in tests/util.py."""
from __future__ import annotations

import contextlib
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from displaced_patch_diffusion_amd import ops, synth
from displaced_patch_diffusion_amd._lib import DPError
from tests.util import assert_close, dev, dev_f32, gpu_ok, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]

R = synth.random_tensor


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@contextlib.contextmanager
def attn_schedule(name):
    """Forces the bf16 attention's work schedule ("split" or "balanced"; None
    leaves the pick to the library) for the workspace query and the call."""
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


# --------------------------------------------------------------------- splice
@pytest.mark.parametrize("dt,B,T_kv,C,t0,T_loc", [
    ("bf16", 2, 1024, 64, 256, 256),
    ("bf16", 2, 4096, 640, 1024, 1024),
    ("f32", 2, 1024, 64, 0, 512),
    ("f32", 3, 100, 5, 37, 41),      # odd sizes: 4-byte path
    ("bf16", 1, 77, 3, 70, 7),       # 2-byte path, band at the end
])
def test_splice_bit_exact(dt, B, T_kv, C, t0, T_loc):
    say("splice", dt, B, T_kv, C, t0, T_loc)
    kb = R(1, "t.kb", (B, T_kv, C), dt)
    vb = R(1, "t.vb", (B, T_kv, C), dt)
    kf = R(2, "t.kf", (B, T_loc, C), dt)
    vf = R(2, "t.vf", (B, T_loc, C), dt)
    ek, ev = oracle.kv_buffer_splice(kb, vb, kf, vf, t0)
    gk, gv = dev(kb, dt), dev(vb, dt)
    gk[:, t0:t0 + T_loc] = float("nan")  # poison: every local row must be rewritten
    ops.dp_kv_buffer_splice(gk, gv, dev(kf, dt), dev(vf, dt), t0)
    torch.cuda.synchronize()
    tdt = torch.int16 if dt == "bf16" else torch.int32
    for g, e in ((gk, ek), (gv, ev)):
        assert torch.equal(g.view(tdt).cpu(), dev(e, dt).view(tdt).cpu())


# --------------------------------------------------------------------- linear
@pytest.mark.parametrize("dt,M,Cin,Cout,bias", [
    ("bf16", 300, 128, 96, True), ("bf16", 1024, 640, 640, False), ("bf16", 129, 64, 32, True),
    ("bf16", 8192, 640, 640, True), ("bf16", 200, 2560, 96, False), ("bf16", 77, 32, 352, True),
    # shapes that select each MFMA tile configuration, every one with a ragged edge
    ("bf16", 24583, 64, 96, True),    # 128x128
    ("bf16", 8229, 128, 96, False),   # 64x128
    ("bf16", 16406, 160, 160, True),  # 160x128
    ("bf16", 16406, 96, 96, False),   # 96x128, 32-wide slices
    ("bf16", 20513, 128, 160, True),  # 128x160
    ("bf16", 20513, 96, 160, False),  # 128x160 with 32-wide slices (K % 64 != 0)
    ("bf16", 9810, 64, 640, True),    # 128x128, five column tiles
    ("bf16", 5000, 96, 640, False),   # 128x128 with 32-wide slices
    ("bf16", 18468, 128, 512, True),  # 160x128, four column tiles
    ("f32", 300, 64, 64, True), ("f32", 77, 50, 30, False),
])
def test_linear(dt, M, Cin, Cout, bias):
    say("linear", dt, M, Cin, Cout, bias)
    x = R(1, "lin.x", (M, Cin), dt)
    w = R(0, "lin.w", (Cout, Cin), dt, Cin ** -0.5)
    b = R(3, "lin.b", (Cout,), "f32", 0.1) if bias else None
    y = ops.dp_linear(dev(x, dt), dev(w, dt), None if b is None else dev_f32(b))
    assert_close(host(y), oracle.linear(x, w, b), dt, "linear")


# ----------------------------------------------------------------------- conv
@pytest.mark.parametrize("dt,B,h,W,Cin,Cout,halos", [
    ("bf16", 2, 5, 9, 64, 64, "both"), ("bf16", 1, 3, 40, 128, 96, "top"),
    ("bf16", 2, 1, 7, 64, 32, "bottom"), ("bf16", 2, 4, 33, 64, 160, "none"),
    ("bf16", 2, 3, 50, 96, 320, "both"), ("bf16", 1, 2, 200, 32, 64, "top"),
    ("bf16", 1, 41, 400, 64, 160, "both"),   # 160x128 tiles, ragged M
    ("bf16", 2, 13, 789, 64, 160, "bottom"), # 128x160 tiles, ragged M
    ("bf16", 1, 41, 451, 64, 512, "both"),   # 160x128 tiles, four column tiles
    ("bf16", 1, 20, 491, 32, 640, "top"),    # 128x128 tiles, 32-wide K slices
    ("f32", 2, 16, 32, 64, 64, "both"), ("f32", 1, 2, 5, 6, 7, "top"),
])
def test_conv3x3(dt, B, h, W, Cin, Cout, halos):
    say("conv", dt, B, h, W, Cin, Cout, halos)
    x = R(1, "conv.x", (B, h, W, Cin), dt)
    w = R(0, "conv.w", (Cout, 3, 3, Cin), dt, (9 * Cin) ** -0.5)
    b = R(3, "conv.b", (Cout,), "f32", 0.1)
    ht = R(2, "conv.ht", (B, W, Cin), dt) if halos in ("both", "top") else None
    hb = R(2, "conv.hb", (B, W, Cin), dt) if halos in ("both", "bottom") else None
    y = ops.dp_conv3x3_stale_halo(dev(x, dt), None if ht is None else dev(ht, dt),
                                  None if hb is None else dev(hb, dt), dev(w, dt), dev_f32(b))
    assert_close(host(y), oracle.conv3x3_halo(x, ht, hb, w, b), dt, "conv")


# ------------------------------------------------------------------ groupnorm
def stale_sums_for(B, T_rem, C, G, N, seed, dt):
    """Stale per-patch sums from synthetic remote activations (the oracle's
    group sums in float64, stored as float32 as the previous step would)."""
    out = np.zeros((N, B, G, 2))
    for p in range(N):
        xr = R(seed, f"gn.remote{p}", (B, T_rem, C), dt)
        out[p] = oracle.group_sums(xr * 1.1 + 0.2, G)
    return out.astype(np.float32)


@pytest.mark.parametrize("dt,B,T,C,G,N,rank,silu,affine", [
    ("bf16", 2, 1024, 640, 32, 4, 1, False, True), ("bf16", 2, 300, 320, 32, 2, 1, True, True),
    ("bf16", 1, 17, 64, 8, 1, 0, False, False), ("f32", 2, 512, 64, 32, 2, 0, False, True),
    ("f32", 2, 100, 12, 4, 3, 2, True, False), ("bf16", 2, 64, 1280, 32, 2, 0, True, True),
    ("bf16", 1, 40, 1024, 1024, 2, 1, False, True),  # one channel per group
    # 16 patches x 32 groups: more stale entries than apply threads, staged by the loop
    ("bf16", 2, 300, 320, 32, 16, 5, True, True),
])
def test_groupnorm(dt, B, T, C, G, N, rank, silu, affine):
    say("gn", dt, B, T, C, G, N, rank, silu, affine)
    x = R(1, "gn.x", (B, T, C), dt)
    st = stale_sums_for(B, T, C, G, N, 2, dt)
    gamma = synth.normal(3, "gn.gamma", (C,), 0.1, 1.0) if affine else None
    beta = synth.normal(3, "gn.beta", (C,), 0.1) if affine else None
    ref, fresh = oracle.groupnorm_stale(x, st, rank, N * T, gamma, beta, 1e-5, silu, G)
    st_dev = dev_f32(st)
    st_dev[rank] = float("nan")  # the rank's own entry is never read
    fresh_dev = torch.empty((B, G, 2), dtype=torch.float32, device="cuda")
    y = ops.dp_groupnorm_stale_stats(dev(x, dt), st_dev, rank, N * T,
                                     None if gamma is None else dev_f32(gamma),
                                     None if beta is None else dev_f32(beta), 1e-5, silu, G,
                                     fresh_sums_out=fresh_dev)
    assert_close(host(y), ref, dt, "groupnorm")
    # fresh sums: float32 accumulation of up to ~1e6 terms, bound 1e-5 * sum|x|
    gf = host(fresh_dev)
    absx = np.abs(x).reshape(B, T, G, C // G).sum((1, 3))
    scale = np.stack([absx, (x * x).reshape(B, T, G, C // G).sum((1, 3))], -1)
    assert (np.abs(gf - fresh) <= 1e-5 * scale + 1e-6).all()


def test_groupnorm_single_patch_null_stale():
    B, T, C, G = 2, 200, 64, 32
    x = R(1, "gn1.x", (B, T, C), "f32")
    ref, _ = oracle.groupnorm_stale(x, np.zeros((1, B, G, 2)), 0, T, None, None, 1e-5, False, G)
    y = ops.dp_groupnorm_stale_stats(dev(x, "f32"), None, 0, T, G=G)
    assert_close(host(y), ref, "f32", "groupnorm n=1")


# ------------------------------------------------------------------ attention
_ATTN_BF16 = [("bf16", 2, 2, 64, 200, 333), ("bf16", 1, 3, 64, 128, 64), ("bf16", 2, 1, 64, 5, 1),
              ("bf16", 1, 2, 64, 257, 1000)]
_ATTN_F32 = [("f32", 2, 2, 32, 512, 1024), ("f32", 1, 3, 64, 100, 77), ("f32", 1, 1, 32, 3, 1)]


# bf16 cases under the planner's pick and each forced schedule; the f32 path
# has one schedule
@pytest.mark.parametrize("dt,B,H,d,Tq,Tkv,schedule",
                         [c + (s,) for c in _ATTN_BF16 for s in (None, "split", "balanced")] +
                         [c + (None,) for c in _ATTN_F32])
def test_attention(dt, B, H, d, Tq, Tkv, schedule):
    say("attn", dt, B, H, d, Tq, Tkv, schedule)
    q = R(1, "at.q", (B, Tq, H * d), dt)
    k = R(1, "at.k", (B, Tkv, H * d), dt)
    v = R(1, "at.v", (B, Tkv, H * d), dt)
    with attn_schedule(schedule):
        out = ops.dp_attn_stale_kv(dev(q, dt), dev(k, dt), dev(v, dt), H)
    assert_close(host(out), oracle.attention(q, k, v, H), dt, "attention")


@pytest.mark.parametrize("Tq,Tkv,qscale", [(130, 700, 3.0), (70, 3001, 4.0), (64, 6000, 2.0), (33, 129, 4.0)])
@pytest.mark.parametrize("schedule", [None, "balanced"])
def test_attention_peaked_scores_bf16(Tq, Tkv, qscale, schedule):
    """Large-magnitude queries: softmax close to one-hot, so later key blocks
    can exceed the first block's max by far and force the reference to move
    (the 6000-key case also splits the key range across blocks)."""
    say("attn peaked", Tq, Tkv, qscale, schedule)
    B, H, d = 1, 2, 64
    q = R(5, "atp.q", (B, Tq, H * d), "bf16", qscale)
    k = R(5, "atp.k", (B, Tkv, H * d), "bf16", 1.0)
    v = R(5, "atp.v", (B, Tkv, H * d), "bf16", 1.0)
    with attn_schedule(schedule):
        out = ops.dp_attn_stale_kv(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), H)
    assert_close(host(out), oracle.attention(q, k, v, H), "bf16", "attention peaked")


@pytest.mark.parametrize("Tq,Tkv,hot", [(64, 300, (128, 192)), (32, 9000, (8500, 8600))])
@pytest.mark.parametrize("schedule", [None, "balanced"])
def test_attention_reference_moves(Tq, Tkv, hot, schedule):
    """A run of identical keys scoring ~69 (log2 units) above every earlier key:
    the kernel must move its softmax reference mid-sequence (rescaling the
    accumulated output, the row sums and the next block's scores already
    issued).  All queries are equal and the hot keys share one value vector,
    so the exact result is that vector (the other keys weigh < 2^-60).  The
    long case also splits the key range, so the partial results carry
    references 2^-69 apart into the combine."""
    say("attn reference moves", Tq, Tkv, hot)
    B, H, d = 1, 2, 64
    q = np.full((B, Tq, H * d), 0.5)
    k = R(6, "atm.k", (B, Tkv, H * d), "bf16", 1.0)
    v = R(6, "atm.v", (B, Tkv, H * d), "bf16", 1.0)
    k[:, hot[0]:hot[1]] = 12.0
    v[:, hot[0]:hot[1]] = v[:, hot[0]]
    ref = oracle.attention(q, k, v, H)
    assert np.allclose(ref, np.broadcast_to(v[:, hot[0]][:, None, :], ref.shape), atol=1e-12)
    with attn_schedule(schedule):
        out = ops.dp_attn_stale_kv(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), H)
    assert_close(host(out), ref, "bf16", "attention reference moves")


@pytest.mark.parametrize("B,H,Tq,Tkv", [
    (1, 1, 128, 128000),   # one unit spread over every resident block: many pieces per unit
    (2, 3, 129, 65),       # fewer (unit, tile) items than blocks: most blocks own nothing
    (2, 10, 1024, 4096),   # SDXL-1024 64x64-level share: units and pieces mixed
    (1, 4, 300, 2049),     # ragged queries and keys inside pieces
])
def test_attention_balanced_schedule(B, H, Tq, Tkv):
    """The balanced schedule, forced on shapes that exercise its bookkeeping:
    segments that start and end inside units, whole units written directly,
    blocks with empty ranges, and the combine of every split unit; the split
    schedule on the same inputs must agree with the oracle too."""
    say("attn balanced", B, H, Tq, Tkv)
    d = 64
    q = R(8, "atb.q", (B, Tq, H * d), "bf16", 2.0)
    k = R(8, "atb.k", (B, Tkv, H * d), "bf16")
    v = R(8, "atb.v", (B, Tkv, H * d), "bf16")
    ref = oracle.attention(q, k, v, H)
    for sched in ("balanced", "split"):
        with attn_schedule(sched):
            out = ops.dp_attn_stale_kv(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), H)
        assert_close(host(out), ref, "bf16", f"attention, {sched} schedule")


def test_attention_schedules_on_seeded_shapes():
    """Both work schedules on 20 seeded random shapes (batch 1-3, 1-6 heads,
    1-1500 queries, 1-6000 keys, plain and peaked queries): sampled rows of
    every case against the oracle."""
    rng = np.random.default_rng(1234)
    for case in range(20):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 7))
        Tq, Tkv = int(rng.integers(1, 1501)), int(rng.integers(1, 6001))
        qs = float(rng.choice([1.0, 3.0]))
        say("attn seeded shape", case, B, H, Tq, Tkv, qs)
        q = R(10 + case, "ats.q", (B, Tq, H * 64), "bf16", qs)
        k = R(10 + case, "ats.k", (B, Tkv, H * 64), "bf16")
        v = R(10 + case, "ats.v", (B, Tkv, H * 64), "bf16")
        rows = sample_rows(Tq, 6, case)
        ref = oracle.attention(q[:, rows], k, v, H)
        for sched in ("split", "balanced"):
            with attn_schedule(sched):
                out = host(ops.dp_attn_stale_kv(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), H))
            assert_close(out[:, rows], ref, "bf16", f"attention case {case}, {sched}")


def test_attention_whole_rounds_then_split():
    """The split schedule with its full rounds run whole and only the last
    round's units split into key chunks (picked for 1000 query blocks on 768
    slots): sampled query rows vs the oracle, from whole units, from split
    units, and at the boundary between them inside one (batch, head)."""
    B, H, Tq, Tkv, d = 2, 2, 32000, 2560, 64
    say("attn whole rounds then split", B, H, Tq, Tkv)
    q = R(9, "atw.q", (B, Tq, H * d), "bf16")
    k = R(9, "atw.k", (B, Tkv, H * d), "bf16")
    v = R(9, "atw.v", (B, Tkv, H * d), "bf16")
    with attn_schedule("split"):
        out = host(ops.dp_attn_stale_kv(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), H))
    # units are (batch, head, 128-query block); with 768 slots the first 768
    # units (batch 0, and batch 1 head 0 plus 18 blocks of head 1) run whole
    rows = np.array(sorted({0, 1, 127, 128, 16383, 17 * 128 - 1, 17 * 128, 18 * 128 - 1, 18 * 128,
                            18 * 128 + 1, 19 * 128, 24000, Tq - 1}))
    assert_close(out[:, rows], oracle.attention(q[:, rows], k, v, H), "bf16", "attention whole + split")


# ---------------------------------------------------------------- error paths
def test_errors_raise_before_launch():
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((32, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(DPError) as e:
        ops.dp_linear(x, w)
    assert e.value.status == 2
    q = torch.zeros((1, 8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(DPError):
        ops.dp_attn_stale_kv(q, q.clone(), q.clone(), 2)  # d = 48


# ------------------------------------------------- limits and degenerate shapes
def test_conv_max_cin_and_beyond():
    """Cin = 2048 is the largest supported bf16 input width (the zero page
    covers one 2048-channel pixel); one more 32-channel step is rejected."""
    say("conv Cin=2048")
    B, h, W, Cin, Cout = 1, 2, 6, 2048, 64
    x = R(1, "cm.x", (B, h, W, Cin), "bf16")
    w = R(0, "cm.w", (Cout, 3, 3, Cin), "bf16", (9 * Cin) ** -0.5)
    ht = R(2, "cm.ht", (B, W, Cin), "bf16")
    y = ops.dp_conv3x3_stale_halo(dev(x, "bf16"), dev(ht, "bf16"), None, dev(w, "bf16"), None)
    assert_close(host(y), oracle.conv3x3_halo(x, ht, None, w, None), "bf16", "conv Cin=2048")
    xb = torch.zeros((1, 1, 4, 2080), dtype=torch.bfloat16, device="cuda")
    wb = torch.zeros((32, 3, 3, 2080), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(DPError) as e:
        ops.dp_conv3x3_stale_halo(xb, None, None, wb, None)
    assert e.value.status == 2


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_groupnorm_max_channels(dt):
    """C = 2048 is the widest supported GroupNorm; C = 4096 is rejected."""
    say("gn C=2048", dt)
    B, T, C, G, N, rank = 2, 50, 2048, 32, 3, 2
    x = R(1, "gm.x", (B, T, C), dt)
    st = stale_sums_for(B, T, C, G, N, 2, dt)
    ref, fresh = oracle.groupnorm_stale(x, st, rank, N * T, None, None, 1e-5, True, G)
    fresh_dev = torch.empty((B, G, 2), dtype=torch.float32, device="cuda")
    y = ops.dp_groupnorm_stale_stats(dev(x, dt), dev_f32(st), rank, N * T, None, None, 1e-5, True, G,
                                     fresh_sums_out=fresh_dev)
    assert_close(host(y), ref, dt, "groupnorm C=2048")
    xb = torch.zeros((1, 4, 4096), dtype=torch.float32 if dt == "f32" else torch.bfloat16, device="cuda")
    with pytest.raises(DPError) as e:
        ops.dp_groupnorm_stale_stats(xb, None, 0, 4, G=32)
    assert e.value.status == 2


@pytest.mark.parametrize("Tq,Tkv", [(1, 20000), (1000, 65), (3, 64)])
@pytest.mark.parametrize("schedule", [None, "balanced"])
def test_attention_degenerate_bf16(Tq, Tkv, schedule):
    """One query against a long (split) key range; many queries against one
    full tile plus one ragged key; fewer queries than one wave's group."""
    say("attn degenerate", Tq, Tkv, schedule)
    B, H, d = 1, 2, 64
    q = R(7, "atd.q", (B, Tq, H * d), "bf16")
    k = R(7, "atd.k", (B, Tkv, H * d), "bf16")
    v = R(7, "atd.v", (B, Tkv, H * d), "bf16")
    with attn_schedule(schedule):
        out = ops.dp_attn_stale_kv(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), H)
    assert_close(host(out), oracle.attention(q, k, v, H), "bf16", "attention degenerate")


def test_linear_single_row_wide_reduction():
    say("linear M=1 Cin=4096")
    x = R(1, "ld.x", (1, 4096), "bf16")
    w = R(0, "ld.w", (96, 4096), "bf16", 4096 ** -0.5)
    b = R(3, "ld.b", (96,), "f32", 0.1)
    y = ops.dp_linear(dev(x, "bf16"), dev(w, "bf16"), dev_f32(b))
    assert_close(host(y), oracle.linear(x, w, b), "bf16", "linear M=1")


def test_splice_whole_buffer():
    """The band covers every token (a single patch): the buffer becomes the
    fresh tensor bit for bit."""
    say("splice whole buffer")
    B, T, C = 2, 300, 64
    kb, vb = R(1, "sw.kb", (B, T, C), "bf16"), R(1, "sw.vb", (B, T, C), "bf16")
    kf, vf = R(2, "sw.kf", (B, T, C), "bf16"), R(2, "sw.vf", (B, T, C), "bf16")
    kd, vd = dev(kb, "bf16"), dev(vb, "bf16")
    ops.dp_kv_buffer_splice(kd, vd, dev(kf, "bf16"), dev(vf, "bf16"), 0)
    assert torch.equal(kd, dev(kf, "bf16")) and torch.equal(vd, dev(vf, "bf16"))


# ----------------------------------------------------- full-size rank shares
BF16_WORKLOADS = [n for n in synth.WORKLOAD_ORDER if synth.WORKLOADS[n].dtype == "bf16"]


def sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    rows = {0, n - 1, n // 2}
    rows |= set(rng.choice(n, size=min(n, k), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", BF16_WORKLOADS)
def test_full_size_share(name):
    """Every op of the share at its real shape: sampled outputs vs the oracle."""
    w = synth.WORKLOADS[name]
    dt, B = w.dtype, w.B
    say("full-size", name)
    # splice + attention at the attention level
    C, Tq, Tkv, t0 = w.attn_C, w.Tq, w.T_kv, w.t0
    kb, vb = R(1, f"{name}.kb", (B, Tkv, C), dt), R(1, f"{name}.vb", (B, Tkv, C), dt)
    kf, vf = R(1, f"{name}.kf", (B, Tq, C), dt), R(1, f"{name}.vf", (B, Tq, C), dt)
    q = R(1, f"{name}.q", (B, Tq, C), dt)
    gk, gv = dev(kb, dt), dev(vb, dt)
    ops.dp_kv_buffer_splice(gk, gv, dev(kf, dt), dev(vf, dt), t0)
    ek, ev = oracle.kv_buffer_splice(kb, vb, kf, vf, t0)
    assert torch.equal(gk.view(torch.int16).cpu(), dev(ek, dt).view(torch.int16).cpu())
    assert torch.equal(gv.view(torch.int16).cpu(), dev(ev, dt).view(torch.int16).cpu())
    out = host(ops.dp_attn_stale_kv(dev(q, dt), gk, gv, w.heads))
    rows = sample_rows(Tq, 12, 7)
    assert_close(out[:, rows], oracle.attention(q[:, rows], ek, ev, w.heads), dt, "attention")
    del gk, gv
    # projection (sampled rows)
    x = R(1, f"{name}.xl", (B, Tq, C), dt)
    wq = R(0, f"{name}.wq", (C, C), dt, C ** -0.5)
    y = host(ops.dp_linear(dev(x, dt), dev(wq, dt)))
    assert_close(y[:, rows], oracle.linear(x[:, rows], wq), dt, "linear")
    # conv (sampled output rows; edge rows included) and GroupNorm at the conv level
    Cc, h, Wd = w.conv_C, w.conv_h, w.conv_W
    xc = R(1, f"{name}.xc", (B, h, Wd, Cc), dt)
    cw = R(0, f"{name}.cw", (Cc, 3, 3, Cc), dt, (9 * Cc) ** -0.5)
    cb = synth.normal(3, f"{name}.cb", (Cc,), 0.1)
    ht = R(2, f"{name}.ht", (B, Wd, Cc), dt)
    hb = R(2, f"{name}.hb", (B, Wd, Cc), dt)
    yc = host(ops.dp_conv3x3_stale_halo(dev(xc, dt), dev(ht, dt), dev(hb, dt), dev(cw, dt), dev_f32(cb)))
    for i in sorted({0, h - 1, h // 2}):
        top = xc[:, i - 1] if i > 0 else ht
        bot = xc[:, i + 1] if i < h - 1 else hb
        ref = oracle.conv3x3_halo(xc[:, i:i + 1], top, bot, cw, cb)
        cols = sample_rows(Wd, 24, i)
        assert_close(yc[:, i:i + 1, cols], ref[:, :, cols], dt, f"conv row {i}")
    T = h * Wd
    st = stale_sums_for(B, T, Cc, w.G, w.N, 2, dt)
    gamma, beta = synth.normal(3, "fg", (Cc,), 0.1, 1.0), synth.normal(3, "fb", (Cc,), 0.1)
    xg = xc.reshape(B, T, Cc)
    ref, _ = oracle.groupnorm_stale(xg, st, w.rank, w.N * T, gamma, beta, w.eps, w.two_level, w.G)
    yg = ops.dp_groupnorm_stale_stats(dev(xg, dt), dev_f32(st), w.rank, w.N * T, dev_f32(gamma),
                                      dev_f32(beta), w.eps, w.two_level, w.G)
    assert_close(host(yg), ref, dt, "groupnorm")


@pytest.mark.parametrize("rank", [0, 7])
def test_full_size_edge_ranks(rank):
    """The SDXL-3840 share of the first and the last row band, at full size, in
    the launch configuration the benchmark times: fused Q/K/V written into the
    buffers at the band's first and last token range (sampled rows vs the
    oracle; rows outside the band untouched), attention over that buffer, and
    the conv whose missing halo is the image edge (zeros, NULL halo)."""
    w = synth.WORKLOADS["sdxl3840_l240_c640"].with_rank(rank)
    dt, B, C, Tq, Tkv, t0 = w.dtype, w.B, w.attn_C, w.Tq, w.T_kv, w.t0
    say("full-size edge rank", rank, "t0", t0)
    x = R(1, f"edge{rank}.x", (B, Tq, C), dt)
    wq, wk, wv = (R(0, f"edge{rank}.w{n}", (C, C), dt, C ** -0.5) for n in "qkv")
    kb, vb = R(1, f"edge{rank}.kb", (B, Tkv, C), dt), R(1, f"edge{rank}.vb", (B, Tkv, C), dt)
    gk, gv = dev(kb, dt), dev(vb, dt)
    q = ops.dp_qkv_projection_into_buffers(dev(x, dt), dev(wq, dt), dev(wk, dt), dev(wv, dt), gk, gv, t0)
    rows = sample_rows(Tq, 8, 11 + rank)
    assert_close(host(q)[:, rows], oracle.linear(x[:, rows], wq), dt, "q")
    hk, hv = host(gk), host(gv)
    assert_close(hk[:, t0 + rows], oracle.linear(x[:, rows], wk), dt, "k rows")
    assert_close(hv[:, t0 + rows], oracle.linear(x[:, rows], wv), dt, "v rows")
    outside = np.r_[0:t0, t0 + Tq:Tkv]
    assert np.array_equal(hk[:, outside], kb[:, outside]) and np.array_equal(hv[:, outside], vb[:, outside])
    # the oracle's buffers: its own projections, stored in the buffers' dtype
    ek, ev = oracle.kv_buffer_splice(kb, vb, synth.as_storage(oracle.linear(x, wk), dt),
                                     synth.as_storage(oracle.linear(x, wv), dt), t0)
    del hk, hv
    out = host(ops.dp_attn_stale_kv(q, gk, gv, w.heads))
    del gk, gv
    assert_close(out[:, rows], oracle.attention(oracle.linear(x[:, rows], wq), ek, ev, w.heads), dt,
                 "attention")
    # conv: the edge rows take zeros for the missing halo
    Cc, h, Wd = w.conv_C, w.conv_h, w.conv_W
    xc = R(1, f"edge{rank}.xc", (B, h, Wd, Cc), dt)
    cw = R(0, f"edge{rank}.cw", (Cc, 3, 3, Cc), dt, (9 * Cc) ** -0.5)
    halo = R(2, f"edge{rank}.halo", (B, Wd, Cc), dt)
    ht, hb = (None, halo) if rank == 0 else (halo, None)
    yc = host(ops.dp_conv3x3_stale_halo(dev(xc, dt), None if ht is None else dev(ht, dt),
                                        None if hb is None else dev(hb, dt), dev(cw, dt), None))
    for i in (0, h - 1):
        top = xc[:, i - 1] if i > 0 else ht
        bot = xc[:, i + 1] if i < h - 1 else hb
        ref = oracle.conv3x3_halo(xc[:, i:i + 1], top, bot, cw, None)
        cols = sample_rows(Wd, 24, i)
        assert_close(yc[:, i:i + 1, cols], ref[:, :, cols], dt, f"conv row {i}")


# ----------------------------------------------------------- whole fp32 chain
def _share_inputs(w, rank):
    """Inputs of one rank's share for the single-level chain: stale K/V from
    the oracle's full-image projection plus stale-step noise, halos from the
    oracle's full-image attention block plus noise, stale GN sums from the
    oracle's full-image chain plus noise on the other patches."""
    w = w.with_rank(rank)
    a = synth.attention_block_inputs(w)
    cv = synth.conv_inputs(w)
    gn = synth.groupnorm_inputs(w)
    B, H, Wd, C = w.B, w.attn_H, w.attn_W, w.attn_C
    x_full = a["x_full"].reshape(B, H * Wd, C)
    k_full = oracle.linear(x_full, a["wk"])
    v_full = oracle.linear(x_full, a["wv"])
    k_buf = synth.as_storage(k_full + a["k_noise"], w.dtype)
    v_buf = synth.as_storage(v_full + a["v_noise"], w.dtype)
    y_full, _, _ = oracle.attention_block_share(x_full, a["wq"], a["wk"], a["wv"], a["wo"],
                                                k_full, v_full, 0, w.heads)
    yimg = y_full.reshape(B, H, Wd, C)
    r0, r1 = w.attn_rows()
    ht = synth.as_storage(yimg[:, r0 - 1] + cv["halo_top_noise"], w.dtype) if r0 > 0 else None
    hb = synth.as_storage(yimg[:, r1] + cv["halo_bot_noise"], w.dtype) if r1 < H else None
    z_full = oracle.conv3x3_halo(synth.as_storage(yimg, w.dtype), None, None, cv["w"], cv["bias"])
    z_full = z_full.reshape(B, H * Wd, C)
    z_noisy = z_full + synth.stale_noise(w, "gn.stale_noise", z_full.shape)
    stale = np.stack([oracle.group_sums(z_noisy[:, w.attn_rows(p)[0] * Wd:w.attn_rows(p)[1] * Wd], w.G)
                      for p in range(w.N)]).astype(np.float32)
    x_loc = np.ascontiguousarray(x_full[:, r0 * Wd:r1 * Wd])
    return dict(x_loc=x_loc, wq=a["wq"], wk=a["wk"], wv=a["wv"], wo=a["wo"], k_buf=k_buf,
                v_buf=v_buf, t0=r0 * Wd, ht=ht, hb=hb, cw=cv["w"], cb=cv["bias"], stale=stale,
                gamma=gn["gamma"], beta=gn["beta"])


def gpu_share_step(w, d):
    """The share on the GPU, every step through the library."""
    dt = w.dtype
    B, C = w.B, w.attn_C
    x = dev(d["x_loc"], dt)
    q = ops.dp_linear(x, dev(d["wq"], dt))
    kf = ops.dp_linear(x, dev(d["wk"], dt))
    vf = ops.dp_linear(x, dev(d["wv"], dt))
    kb, vb = dev(d["k_buf"], dt), dev(d["v_buf"], dt)
    ops.dp_kv_buffer_splice(kb, vb, kf, vf, d["t0"])
    o = ops.dp_attn_stale_kv(q, kb, vb, w.heads)
    y = ops.dp_linear(o, dev(d["wo"], dt))
    h = w.Tq // w.attn_W
    z = ops.dp_conv3x3_stale_halo(y.view(B, h, w.attn_W, C),
                                  None if d["ht"] is None else dev(d["ht"], dt),
                                  None if d["hb"] is None else dev(d["hb"], dt),
                                  dev(d["cw"], dt), dev_f32(d["cb"]))
    fresh = torch.empty((B, w.G, 2), dtype=torch.float32, device="cuda")
    out = ops.dp_groupnorm_stale_stats(z.view(B, w.Tq, C), dev_f32(d["stale"]), w.rank,
                                       w.T_kv, dev_f32(d["gamma"]), dev_f32(d["beta"]), w.eps,
                                       False, w.G, fresh_sums_out=fresh)
    return out, fresh


@pytest.mark.parametrize("rank", [0, 1])
def test_fp32_share_chain(rank):
    """Whole rank share of the tiny fp32 workload vs the oracle's chain."""
    w = synth.WORKLOADS["tiny32_c64_fp32"].with_rank(rank)
    say("chain fp32 rank", rank)
    d = _share_inputs(w, rank)
    ref = oracle.rank_share_step(d["x_loc"], d["wq"], d["wk"], d["wv"], d["wo"], d["k_buf"],
                                 d["v_buf"], d["t0"], w.heads, w.attn_W, d["ht"], d["hb"], d["cw"],
                                 d["cb"], d["stale"], rank, w.T_kv, d["gamma"], d["beta"], w.eps,
                                 w.G)
    out, fresh = gpu_share_step(w, d)
    assert_close(host(out), ref["out"], "f32", "chain out")
    assert_close(host(fresh), ref["fresh_sums"], "f32", "chain fresh sums")


def test_stale_equals_fresh_ranks_concat_on_gpu():
    """Noise zero: the GPU shares of all ranks concatenate to the GPU's own
    single-patch (N=1) result -- a property that holds at any size."""
    w = synth.WORKLOADS["sdxl1024_l64_c640"].with_noise(0.0)
    dt, B, C, Wd, Hh = w.dtype, w.B, w.attn_C, w.attn_W, w.attn_H
    a = synth.attention_block_inputs(w)
    x_full = dev(a["x_full"].reshape(B, Hh * Wd, C), dt)
    wq, wk, wv = dev(a["wq"], dt), dev(a["wk"], dt), dev(a["wv"], dt)
    k_full, v_full = ops.dp_linear(x_full, wk), ops.dp_linear(x_full, wv)
    ref = ops.dp_attn_stale_kv(ops.dp_linear(x_full, wq), k_full, v_full, w.heads)
    parts = []
    for r in range(w.N):
        r0, r1 = w.attn_rows(r)
        xl = x_full[:, r0 * Wd:r1 * Wd].contiguous()
        kb, vb = k_full.clone(), v_full.clone()
        kb[:, r0 * Wd:r1 * Wd] = 0
        ops.dp_kv_buffer_splice(kb, vb, ops.dp_linear(xl, wk), ops.dp_linear(xl, wv), r0 * Wd)
        parts.append(ops.dp_attn_stale_kv(ops.dp_linear(xl, wq), kb, vb, w.heads))
    cat = torch.cat(parts, 1)
    # The key-chunk split chosen for the full image (4096 queries) differs from
    # the one for a share (1024 queries), so the summation order differs: the
    # property holds to the bf16 tolerance, not bit for bit.
    assert_close(host(cat), host(ref), "bf16", "stale==fresh concatenation")
    # and both equal the oracle's unsplit attention of the full image (float64
    # projections from the same inputs) on one query row per 128-query block
    xf = a["x_full"].reshape(B, Hh * Wd, C)
    rows = np.arange(17, Hh * Wd, 128)
    ref_o = oracle.attention(oracle.linear(xf[:, rows], a["wq"]), oracle.linear(xf, a["wk"]),
                             oracle.linear(xf, a["wv"]), w.heads)
    assert_close(host(cat)[:, rows], ref_o, "bf16", "stale==fresh concatenation vs oracle")


# ------------------------------------------- fused Q/K/V projection (NEXT-2)
@pytest.mark.parametrize("dt,B,T_kv,C,t0,T_loc", [
    ("bf16", 2, 1000, 640, 300, 200), ("bf16", 1, 96, 64, 0, 96), ("bf16", 2, 333, 320, 250, 83),
    ("bf16", 2, 8000, 640, 900, 7100),  # the 160x128 tiles of the SDXL-3840 share
    ("f32", 2, 256, 64, 64, 64), ("f32", 1, 50, 12, 40, 10),
])
def test_qkv_projection_into_buffers(dt, B, T_kv, C, t0, T_loc):
    """Equals dp_linear x3 + dp_kv_buffer_splice bit for bit (rows outside
    the band untouched), and the oracle's projections within tolerance."""
    say("qkv fused", dt, B, T_kv, C, t0, T_loc)
    x = R(1, "qkv.x", (B, T_loc, C), dt)
    ws = [R(0, f"qkv.w{i}", (C, C), dt, C ** -0.5) for i in range(3)]
    kb, vb = R(2, "qkv.kb", (B, T_kv, C), dt), R(2, "qkv.vb", (B, T_kv, C), dt)
    xd, wd = dev(x, dt), [dev(w, dt) for w in ws]
    k1, v1 = dev(kb, dt), dev(vb, dt)
    q1 = ops.dp_qkv_projection_into_buffers(xd, wd[0], wd[1], wd[2], k1, v1, t0)
    k2, v2 = dev(kb, dt), dev(vb, dt)
    q2 = ops.dp_linear(xd, wd[0])
    ops.dp_kv_buffer_splice(k2, v2, ops.dp_linear(xd, wd[1]), ops.dp_linear(xd, wd[2]), t0)
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    assert_close(host(q1), oracle.linear(x, ws[0]), dt, "fused q")
    assert_close(host(k1[:, t0:t0 + T_loc]), oracle.linear(x, ws[1]), dt, "fused k")
    assert_close(host(v1[:, t0:t0 + T_loc]), oracle.linear(x, ws[2]), dt, "fused v")
    outside = np.r_[0:t0, t0 + T_loc:T_kv]
    assert np.array_equal(host(k1)[:, outside], np.asarray(kb, np.float64)[:, outside])
