"""Pins for the CPU oracle: each test ties it to something other than itself.

* library special cases: with one patch (or with stale == fresh, concatenated
  over all ranks) each displaced op must equal the unsplit op, computed here by
  torch's float64 CPU routines (scaled_dot_product_attention, conv2d,
  group_norm, silu) -- routines the oracle never calls;
* closed forms and invariants (softmax rows summing to one, a single key, zero
  keys, a delta kernel, shifted taps, constant inputs, clamped variance);
* facts the pages print (row-band seams, tests/golden/partition_seams.json) and
  the pages' splice rule (local slice exactly fresh, remote never a blend:
  "OTIL for SDXL on 4x L40S", "Self-tests").
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


# ------------------------------------------------------------------ partition
def test_partition_seams_match_pages():
    with open(os.path.join(GOLDEN, "partition_seams.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        H, N = c["H"], c["N"]
        bands = [oracle.partition_rows(H, N, r) for r in range(N)]
        assert bands[0][0] == 0 and bands[-1][1] == H
        assert all(bands[r][1] == bands[r + 1][0] for r in range(N - 1))
        seams = [bands[r][1] for r in range(N - 1)]
        assert len(seams) == c["n_seams"]
        if "seams" in c:
            assert seams == c["seams"]


@pytest.mark.parametrize("H,N", [(240, 8), (7, 3), (5, 5), (1, 1)])
def test_partition_covers_rows_once(H, N):
    cover = np.zeros(H, dtype=int)
    for r in range(N):
        r0, r1 = oracle.partition_rows(H, N, r)
        assert r1 - r0 in (H // N, H // N + 1)
        cover[r0:r1] += 1
    assert (cover == 1).all()


# --------------------------------------------------------------------- linear
def test_linear_matches_matmul():
    x, w, b = rnd(1, 3, 5, 17), rnd(2, 9, 17), rnd(3, 9)
    np.testing.assert_allclose(oracle.linear(x, w, b), x @ w.T + b, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.linear(x, w), x @ w.T, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------- splice
def test_splice_rule_local_fresh_remote_untouched():
    B, T, C, t0, Tl = 2, 20, 6, 8, 5
    k = rnd(4, B, T, C).astype(np.float32)
    v = rnd(5, B, T, C).astype(np.float32)
    k[:, t0:t0 + Tl] = np.nan  # poison the local rows: they must all be replaced
    kf, vf = rnd(6, B, Tl, C).astype(np.float32), rnd(7, B, Tl, C).astype(np.float32)
    ks, vs = oracle.kv_buffer_splice(k, v, kf, vf, t0)
    assert np.array_equal(ks[:, t0:t0 + Tl].view(np.uint32), kf.view(np.uint32))
    assert np.array_equal(vs[:, t0:t0 + Tl].view(np.uint32), vf.view(np.uint32))
    rest = np.r_[0:t0, t0 + Tl:T]
    assert np.array_equal(ks[:, rest].view(np.uint32), k[:, rest].view(np.uint32))
    assert np.array_equal(vs[:, rest].view(np.uint32), v[:, rest].view(np.uint32))
    assert not np.isnan(ks).any()


# ------------------------------------------------------------------ attention
def sdpa(q, k, v, heads, scale=None):
    B, Tq, C = q.shape
    d = C // heads
    f = lambda a: t64(a).reshape(a.shape[0], a.shape[1], heads, d).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(f(q), f(k), f(v), scale=scale)
    return o.permute(0, 2, 1, 3).reshape(B, Tq, C).numpy()


@pytest.mark.parametrize("B,H,Tq,Tkv,d", [(2, 2, 7, 13, 32), (1, 3, 5, 40, 64), (2, 1, 1, 1, 16),
                                          (1, 2, 33, 65, 8)])
def test_attention_matches_torch_sdpa(B, H, Tq, Tkv, d):
    q, k, v = rnd(10, B, Tq, H * d), rnd(11, B, Tkv, H * d), rnd(12, B, Tkv, H * d)
    np.testing.assert_allclose(oracle.attention(q, k, v, H), sdpa(q, k, v, H), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(oracle.attention(q, k, v, H, 0.3), sdpa(q, k, v, H, 0.3),
                               rtol=1e-11, atol=1e-12)


def test_attention_rows_sum_to_one():
    # V = one-hot rows makes the output the softmax matrix itself.
    B, H, Tq, d = 2, 2, 9, 16
    Tkv = d
    q, k = rnd(13, B, Tq, H * d, std=2.0), rnd(14, B, Tkv, H * d, std=2.0)
    v = np.tile(np.eye(d), (B, 1, H)).reshape(B, Tkv, H * d)
    P = oracle.attention(q, k, v, H).reshape(B, Tq, H, d)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (P > 0).all() and (P < 1).all()


def test_attention_closed_forms():
    B, H, Tq, d = 1, 2, 4, 8
    q = rnd(15, B, Tq, H * d)
    # a single key: the output is that key's value
    k1, v1 = rnd(16, B, 1, H * d), rnd(17, B, 1, H * d)
    np.testing.assert_allclose(oracle.attention(q, k1, v1, H), np.broadcast_to(v1, q.shape), atol=1e-14)
    # all-zero keys: uniform weights, the output is the mean value
    v = rnd(18, B, 11, H * d)
    np.testing.assert_allclose(oracle.attention(q, np.zeros((B, 11, H * d)), v, H),
                               np.broadcast_to(v.mean(1, keepdims=True), q.shape), atol=1e-14)
    # two keys: the weight of key 0 is the logistic function of the score gap
    k2, v2 = rnd(19, B, 2, H * d), rnd(20, B, 2, H * d)
    o = oracle.attention(q, k2, v2, H).reshape(B, Tq, H, d)
    qh, kh, vh = q.reshape(B, Tq, H, d), k2.reshape(B, 2, H, d), v2.reshape(B, 2, H, d)
    gap = ((qh * kh[:, None, 0]).sum(-1) - (qh * kh[:, None, 1]).sum(-1)) / np.sqrt(d)
    w0 = 1.0 / (1.0 + np.exp(-gap))
    expect = w0[..., None] * vh[:, None, 0] + (1 - w0[..., None]) * vh[:, None, 1]
    np.testing.assert_allclose(o, expect, atol=1e-13)


def test_attention_output_in_value_hull():
    B, H, Tq, Tkv, d = 2, 2, 6, 30, 8
    q, k, v = rnd(21, B, Tq, H * d, std=3), rnd(22, B, Tkv, H * d), rnd(23, B, Tkv, H * d)
    o = oracle.attention(q, k, v, H)
    assert (o <= v.max(1, keepdims=True) + 1e-12).all() and (o >= v.min(1, keepdims=True) - 1e-12).all()


def test_attention_block_stale_equals_fresh_concat():
    """With stale == fresh, the per-rank shares concatenate to the unsplit block
    (DistriFusion summary, "How It Works": the synchronous first step)."""
    B, Hi, Wd, C, heads, N = 2, 8, 4, 16, 2, 4
    x = rnd(24, B, Hi * Wd, C)
    wq, wk, wv, wo = (rnd(25 + i, C, C, std=C ** -0.5) for i in range(4))
    full = sdpa(x @ wq.T, x @ wk.T, x @ wv.T, heads) @ wo.T  # unsplit, via torch
    k_full, v_full = x @ wk.T, x @ wv.T
    parts = []
    for r in range(N):
        r0, r1 = oracle.partition_rows(Hi, N, r)
        xl = x[:, r0 * Wd:r1 * Wd]
        kb, vb = k_full.copy(), v_full.copy()
        kb[:, r0 * Wd:r1 * Wd] = 1e3  # local rows must come from the splice
        y, _, _ = oracle.attention_block_share(xl, wq, wk, wv, wo, kb, vb, r0 * Wd, heads)
        parts.append(y)
    np.testing.assert_allclose(np.concatenate(parts, 1), full, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------- conv
def torch_conv(xpad_rows, w, b, pad_rows):
    """NHWC in, NHWC out; columns always zero-padded by one."""
    xt = t64(xpad_rows).permute(0, 3, 1, 2)
    wt = t64(w).permute(0, 3, 1, 2)
    y = F.conv2d(xt, wt, None if b is None else t64(b), padding=(pad_rows, 1))
    return y.permute(0, 2, 3, 1).numpy()


@pytest.mark.parametrize("B,h,W,Cin,Cout", [(2, 5, 7, 6, 4), (1, 1, 3, 8, 5), (1, 3, 1, 2, 3)])
def test_conv_no_halo_matches_conv2d(B, h, W, Cin, Cout):
    x, w, b = rnd(30, B, h, W, Cin), rnd(31, Cout, 3, 3, Cin), rnd(32, Cout)
    np.testing.assert_allclose(oracle.conv3x3_halo(x, None, None, w, b), torch_conv(x, w, b, 1),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("h", [1, 2, 6])
def test_conv_halo_matches_conv2d_on_extended_rows(h):
    B, W, Cin, Cout = 2, 5, 4, 3
    x, w, b = rnd(33, B, h, W, Cin), rnd(34, Cout, 3, 3, Cin), rnd(35, Cout)
    ht, hb = rnd(36, B, W, Cin), rnd(37, B, W, Cin)
    ext = np.concatenate([ht[:, None], x, hb[:, None]], 1)
    np.testing.assert_allclose(oracle.conv3x3_halo(x, ht, hb, w, b), torch_conv(ext, w, b, 0),
                               rtol=1e-12, atol=1e-12)
    # a NULL halo reads as zeros
    ext0 = np.concatenate([np.zeros_like(ht[:, None]), x, hb[:, None]], 1)
    np.testing.assert_allclose(oracle.conv3x3_halo(x, None, hb, w, b), torch_conv(ext0, w, b, 0),
                               rtol=1e-12, atol=1e-12)


def test_conv_closed_forms():
    B, h, W, C = 1, 4, 5, 3
    x = rnd(38, B, h, W, C)
    ht, hb = rnd(39, B, W, C), rnd(40, B, W, C)
    eye = np.eye(C)

    def tap(dy, dx):
        w = np.zeros((C, 3, 3, C))
        w[:, dy, dx, :] = eye
        return w

    # centre delta: identity
    np.testing.assert_array_equal(oracle.conv3x3_halo(x, ht, hb, tap(1, 1)), x)
    # tap above: y[i] = x[i-1], row 0 takes halo_top
    y = oracle.conv3x3_halo(x, ht, hb, tap(0, 1))
    np.testing.assert_array_equal(y[:, 0], ht)
    np.testing.assert_array_equal(y[:, 1:], x[:, :-1])
    # tap below: y[i] = x[i+1], last row takes halo_bot
    y = oracle.conv3x3_halo(x, ht, hb, tap(2, 1))
    np.testing.assert_array_equal(y[:, -1], hb)
    np.testing.assert_array_equal(y[:, :-1], x[:, 1:])
    # tap left: y[., j] = x[., j-1], column 0 is zero padding
    y = oracle.conv3x3_halo(x, ht, hb, tap(1, 0))
    np.testing.assert_array_equal(y[:, :, 0], 0)
    np.testing.assert_array_equal(y[:, :, 1:], x[:, :, :-1])
    # all-zero band: only the edge rows see the halos
    w = rnd(41, C, 3, 3, C)
    y = oracle.conv3x3_halo(np.zeros_like(x), ht, hb, w)
    assert np.abs(y[:, 1:-1]).max() == 0 and np.abs(y[:, 0]).max() > 0 and np.abs(y[:, -1]).max() > 0


def test_conv_stale_equals_fresh_concat():
    B, Hi, W, C, Co, N = 2, 12, 5, 4, 3, 3
    x, w, b = rnd(42, B, Hi, W, C), rnd(43, Co, 3, 3, C), rnd(44, Co)
    full = torch_conv(x, w, b, 1)
    parts = []
    for r in range(N):
        r0, r1 = oracle.partition_rows(Hi, N, r)
        ht = x[:, r0 - 1] if r0 > 0 else None
        hb = x[:, r1] if r1 < Hi else None
        parts.append(oracle.conv3x3_halo(x[:, r0:r1], ht, hb, w, b))
    np.testing.assert_allclose(np.concatenate(parts, 1), full, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ groupnorm
def torch_gn(x, G, gamma, beta, eps):
    xt = t64(x).permute(0, 2, 1)
    y = F.group_norm(xt, G, None if gamma is None else t64(gamma),
                     None if beta is None else t64(beta), eps)
    return y.permute(0, 2, 1).numpy()


def numpy_group_sums(x, G):
    B, T, C = x.shape
    xr = x.reshape(B, T, G, C // G)
    return np.stack([xr.sum((1, 3)), (xr * xr).sum((1, 3))], -1)


@pytest.mark.parametrize("B,T,C,G", [(2, 9, 64, 32), (1, 17, 20, 4), (2, 3, 12, 12)])
def test_groupnorm_single_patch_matches_torch(B, T, C, G):
    x = rnd(50, B, T, C, std=2) + 0.5
    gamma, beta = 1 + rnd(51, C, std=0.1), rnd(52, C, std=0.1)
    st = np.zeros((1, B, G, 2))
    y, fresh = oracle.groupnorm_stale(x, st, 0, T, gamma, beta, 1e-5, False, G)
    np.testing.assert_allclose(y, torch_gn(x, G, gamma, beta, 1e-5), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(fresh, numpy_group_sums(x, G), rtol=1e-12, atol=1e-12)
    ys, _ = oracle.groupnorm_stale(x, st, 0, T, gamma, beta, 1e-5, True, G)
    silu = F.silu(t64(torch_gn(x, G, gamma, beta, 1e-5))).numpy()
    np.testing.assert_allclose(ys, silu, rtol=1e-11, atol=1e-11)


def test_groupnorm_stale_equals_fresh_concat():
    B, Hi, W, C, G, N = 2, 8, 3, 16, 4, 4
    x = rnd(53, B, Hi * W, C) * 1.5 - 0.3
    gamma, beta = 1 + rnd(54, C, std=0.1), rnd(55, C, std=0.1)
    full = torch_gn(x, G, gamma, beta, 1e-5)
    bands = [oracle.partition_rows(Hi, N, r) for r in range(N)]
    stale = np.stack([numpy_group_sums(x[:, r0 * W:r1 * W], G) for r0, r1 in bands])
    parts = []
    for r, (r0, r1) in enumerate(bands):
        st = stale.copy()
        st[r] = np.nan  # the rank's own entry must never be read
        y, fresh = oracle.groupnorm_stale(x[:, r0 * W:r1 * W], st, r, Hi * W, gamma, beta, 1e-5, False, G)
        np.testing.assert_allclose(fresh, stale[r], rtol=1e-12, atol=1e-12)
        parts.append(y)
    cat = np.concatenate(parts, 1)
    np.testing.assert_allclose(cat, full, rtol=1e-10, atol=1e-11)
    # gamma=1, beta=0: every (b, g) has mean 0 and variance var/(var+eps)
    y1 = np.concatenate([oracle.groupnorm_stale(x[:, r0 * W:r1 * W], stale, r, Hi * W, None, None,
                                                1e-5, False, G)[0] for r, (r0, r1) in enumerate(bands)], 1)
    xr, yr = x.reshape(B, -1, G, C // G), y1.reshape(B, -1, G, C // G)
    var = xr.var((1, 3))
    np.testing.assert_allclose(yr.mean((1, 3)), 0, atol=1e-12)
    np.testing.assert_allclose(yr.var((1, 3)), var / (var + 1e-5), rtol=1e-10)


def test_groupnorm_closed_forms():
    B, T, C, G = 1, 6, 8, 2
    gamma, beta = 1 + rnd(56, C, std=0.1), rnd(57, C, std=0.1)
    # constant input, no other patches: zero variance, output is beta
    y, _ = oracle.groupnorm_stale(np.full((B, T, C), 3.25), np.zeros((1, B, G, 2)), 0, T, gamma, beta,
                                  1e-5, False, G)
    np.testing.assert_allclose(y, np.broadcast_to(beta, y.shape), atol=1e-12)
    # constant local patch a plus one stale patch with known sums
    a, S1, S2, Tr = 0.75, 13.0, 60.0, 10
    n_loc, n = T * (C // G), (T + Tr) * (C // G)
    st = np.zeros((2, B, G, 2))
    st[1, :, :, 0], st[1, :, :, 1] = S1, S2
    mean = (a * n_loc + S1) / n
    var = (a * a * n_loc + S2) / n - mean ** 2
    y, _ = oracle.groupnorm_stale(np.full((B, T, C), a), st, 0, T + Tr, None, None, 1e-5, False, G)
    np.testing.assert_allclose(y, (a - mean) / np.sqrt(var + 1e-5), rtol=1e-13)
    # inconsistent stale sums (S2/n < mean^2): variance clamps to zero
    st[1, :, :, 1] = 0.0
    mean = (a * n_loc + S1) / n
    assert (a * a * n_loc) / n - mean ** 2 < 0
    y, _ = oracle.groupnorm_stale(np.full((B, T, C), a), st, 0, T + Tr, None, None, 1e-5, False, G)
    np.testing.assert_allclose(y, (a - mean) / np.sqrt(1e-5), rtol=1e-13)


# ---------------------------------------------------------------------- chain
def test_rank_share_step_stale_equals_fresh_concat():
    """Whole share (attention block, conv with halos, GroupNorm with stale
    sums), noise zero: the ranks' outputs concatenate to the unsplit chain,
    which is computed here entirely with torch routines."""
    B, Hi, W, C, heads, N, G = 2, 8, 4, 32, 2, 4, 8
    x = rnd(60, B, Hi * W, C)
    wq, wk, wv, wo = (rnd(61 + i, C, C, std=C ** -0.5) for i in range(4))
    cw, cb = rnd(65, C, 3, 3, C, std=(9 * C) ** -0.5), rnd(66, C, std=0.1)
    gamma, beta = 1 + rnd(67, C, std=0.1), rnd(68, C, std=0.1)
    y_full = sdpa(x @ wq.T, x @ wk.T, x @ wv.T, heads) @ wo.T
    z_full = torch_conv(y_full.reshape(B, Hi, W, C), cw, cb, 1).reshape(B, Hi * W, C)
    out_full = torch_gn(z_full, G, gamma, beta, 1e-5)
    bands = [oracle.partition_rows(Hi, N, r) for r in range(N)]
    stale = np.stack([numpy_group_sums(z_full[:, r0 * W:r1 * W], G) for r0, r1 in bands])
    yimg = y_full.reshape(B, Hi, W, C)
    outs = []
    for r, (r0, r1) in enumerate(bands):
        res = oracle.rank_share_step(
            x[:, r0 * W:r1 * W], wq, wk, wv, wo, x @ wk.T, x @ wv.T, r0 * W, heads, W,
            yimg[:, r0 - 1] if r0 > 0 else None, yimg[:, r1] if r1 < Hi else None,
            cw, cb, stale, r, Hi * W, gamma, beta, 1e-5, G)
        outs.append(res["out"])
    np.testing.assert_allclose(np.concatenate(outs, 1), out_full, rtol=1e-9, atol=1e-10)


# ------------------------------------------------------- multi-step schedule
def _schedule_weights(C, seed=70):
    return {"wq": rnd(seed, C, C, std=C ** -0.5), "wk": rnd(seed + 1, C, C, std=C ** -0.5),
            "wv": rnd(seed + 2, C, C, std=C ** -0.5), "wo": rnd(seed + 3, C, C, std=C ** -0.5),
            "conv_w": rnd(seed + 4, C, 3, 3, C, std=(9 * C) ** -0.5), "conv_b": rnd(seed + 5, C, std=0.1),
            "gamma": 1 + rnd(seed + 6, C, std=0.1), "beta": rnd(seed + 7, C, std=0.1)}


def _torch_chain(x, w, B, Hi, W, C, heads, G):
    y = sdpa(x @ w["wq"].T, x @ w["wk"].T, x @ w["wv"].T, heads) @ w["wo"].T
    z = torch_conv(y.reshape(B, Hi, W, C), w["conv_w"], w["conv_b"], 1).reshape(B, Hi * W, C)
    return torch_gn(z, G, w["gamma"], w["beta"], 1e-5)


@pytest.mark.parametrize("N", [1, 4])
def test_schedule_sync_steps_equal_unsplit_chain(N):
    """Synchronous steps ("DistriFusion" summary, "How It Works": the first
    step is synchronous) over N bands equal the unsplit chain, computed by
    torch, applied step after step."""
    B, Hi, W, C, heads, G = 2, 8, 4, 16, 2, 4
    w = _schedule_weights(C)
    sch = oracle.DisplacedSchedule(Hi, W, heads, N, w, G=G)
    x = ref = rnd(80, B, Hi * W, C)
    for _ in range(3):
        x = sch.step(x, True)
        ref = _torch_chain(ref, w, B, Hi, W, C, heads, G)
        np.testing.assert_allclose(x, ref, rtol=1e-9, atol=1e-10)


def test_schedule_single_band_displaced_equals_sync():
    """With one band nothing is stale: displaced steps equal the chain."""
    B, Hi, W, C, heads, G = 1, 6, 4, 16, 2, 4
    w = _schedule_weights(C, 90)
    sch = oracle.DisplacedSchedule(Hi, W, heads, 1, w, G=G)
    x = ref = rnd(91, B, Hi * W, C)
    for s in range(3):
        x = sch.step(x, s == 0)
        ref = _torch_chain(ref, w, B, Hi, W, C, heads, G)
        np.testing.assert_allclose(x, ref, rtol=1e-9, atol=1e-10)


def test_schedule_displaced_with_unchanged_input_equals_sync():
    """When the activations did not change between steps, the state recorded
    one step earlier is the current state, so a displaced step reproduces the
    synchronous one."""
    B, Hi, W, C, heads, G, N = 2, 8, 4, 16, 2, 4, 4
    w = _schedule_weights(C, 100)
    x = rnd(101, B, Hi * W, C)
    sch = oracle.DisplacedSchedule(Hi, W, heads, N, w, G=G)
    sync_out = sch.step(x, True)
    disp_out = sch.step(x, False)
    np.testing.assert_allclose(disp_out, sync_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(disp_out, _torch_chain(x, w, B, Hi, W, C, heads, G), rtol=1e-9, atol=1e-10)


def test_schedule_displaced_step_reads_other_bands_from_previous_step():
    """In a displaced step, band r's output depends on the other bands' current
    activations only through the previous step's state: perturbing band p's
    input right before the step changes band p's output and no other band's.
    A synchronous step propagates the perturbation."""
    B, Hi, W, C, heads, G, N = 1, 8, 4, 16, 2, 4, 4
    w = _schedule_weights(C, 110)
    x0 = rnd(111, B, Hi * W, C)
    p = 2
    r0, r1 = oracle.partition_rows(Hi, N, p)
    for sync in (False, True):
        outs = []
        for delta in (0.0, 0.5):
            sch = oracle.DisplacedSchedule(Hi, W, heads, N, w, G=G)
            x1 = sch.step(x0, True)
            x1[:, r0 * W:r1 * W] += delta
            outs.append(sch.step(x1, sync))
        changed = np.abs(outs[0] - outs[1]).reshape(B, Hi, W, C).max(axis=(0, 2, 3)) > 0
        if sync:
            assert changed.sum() > r1 - r0  # other bands see the perturbation
        else:
            assert changed[r0:r1].all() and not changed[:r0].any() and not changed[r1:].any()


def test_schedule_sampler_update_single_band_equals_torch():
    """The sampler update x + alpha (stack(x) - x) between steps, one band
    (nothing stale): equal to the torch chain blended the same way."""
    B, Hi, W, C, heads, G, a = 1, 6, 4, 16, 2, 4, 0.3
    w = _schedule_weights(C, 120)
    sch = oracle.DisplacedSchedule(Hi, W, heads, 1, w, G=G)
    x = ref = rnd(121, B, Hi * W, C)
    for s in range(3):
        x = sch.step(x, s == 0, a)
        ref = ref + a * (_torch_chain(ref, w, B, Hi, W, C, heads, G) - ref)
        np.testing.assert_allclose(x, ref, rtol=1e-9, atol=1e-10)
