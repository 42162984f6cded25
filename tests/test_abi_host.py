"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/dp.h declares, and rejects bad arguments before any
device work (so these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

from displaced_patch_diffusion_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dp.h")

# Fake, far-apart device addresses: validation rejects the call before any use.
A, Bp, Cp, D, E = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(dp_[a-z0-9_]+)\s*\(", src))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libdp.so is not built (python -m displaced_patch_diffusion_amd.build)")
    return _lib.lib()


def test_exports_every_declared_symbol(lib):
    names = declared()
    assert {"dp_kv_buffer_splice", "dp_attn_stale_kv", "dp_conv3x3_stale_halo",
            "dp_groupnorm_stale_stats", "dp_linear"} <= names
    assert names == set(_lib.SIGNATURES), "binding signature table out of sync with the header"
    cdll = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(cdll, n), n


def test_status_strings(lib):
    for s in range(4):
        assert lib.dp_status_string(s)
    assert lib.dp_status_string(99) == b"unknown status"


def status_and_error(fn, *args):
    st = fn(*args)
    return st, _lib.lib().dp_last_error().decode()


def test_splice_validation(lib):
    st, msg = status_and_error(lib.dp_kv_buffer_splice, None, Bp, Cp, D, 2, 16, 8, 0, 4, 1, None)
    assert st == _lib.DP_ERR_INVALID_ARG and "NULL" in msg
    st, msg = status_and_error(lib.dp_kv_buffer_splice, A, Bp, Cp, D, 2, 16, 8, 13, 4, 1, None)
    assert st == _lib.DP_ERR_INVALID_ARG and "outside" in msg
    st, _ = status_and_error(lib.dp_kv_buffer_splice, A, Bp, Cp, D, 2, 16, 8, -1, 4, 1, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    st, _ = status_and_error(lib.dp_kv_buffer_splice, A, Bp, Cp, D, 0, 16, 8, 0, 4, 1, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    # fresh rows inside the buffer they are spliced into
    st, msg = status_and_error(lib.dp_kv_buffer_splice, A, Bp, A + 64, D, 2, 16, 8, 0, 4, 1, None)
    assert st == _lib.DP_ERR_INVALID_ARG and "overlap" in msg
    st, _ = status_and_error(lib.dp_kv_buffer_splice, A, Bp, Cp, D, 2, 16, 8, 0, 4, 7, None)
    assert st == _lib.DP_ERR_INVALID_ARG


def test_attention_validation(lib):
    ws0 = lib.dp_attn_stale_kv_workspace(2, 10, 1024, 4096, 64, _lib.DP_BF16)
    assert ws0 >= 0
    args = [A, Bp, Cp, D, 2, 10, 100, 300]
    st, _ = status_and_error(lib.dp_attn_stale_kv, None, *args[1:], 64, 0.0, 1, None, 0, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    st, msg = status_and_error(lib.dp_attn_stale_kv, *args, 48, 0.0, _lib.DP_BF16, None, 0, None)
    assert st == _lib.DP_ERR_UNSUPPORTED and "head dim" in msg
    st, _ = status_and_error(lib.dp_attn_stale_kv, *args, 128, 0.0, _lib.DP_F32, None, 0, None)
    assert st == _lib.DP_ERR_UNSUPPORTED
    st, _ = status_and_error(lib.dp_attn_stale_kv, A, Bp, Cp, D, 2, 10, 0, 300, 64, 0.0, 1, None, 0, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    st, msg = status_and_error(lib.dp_attn_stale_kv, A, Bp, Cp, A + 2, 2, 10, 100, 300, 64, 0.0, 1, None, 0, None)
    assert st == _lib.DP_ERR_INVALID_ARG and "overlap" in msg


def _attn_ws(lib, schedule, B, H, Tq, Tkv):
    old = os.environ.get("DP_ATTN_SCHEDULE")
    if schedule is None:
        os.environ.pop("DP_ATTN_SCHEDULE", None)
    else:
        os.environ["DP_ATTN_SCHEDULE"] = schedule
    try:
        return lib.dp_attn_stale_kv_workspace(B, H, Tq, Tkv, 64, _lib.DP_BF16)
    finally:
        if old is None:
            os.environ.pop("DP_ATTN_SCHEDULE", None)
        else:
            os.environ["DP_ATTN_SCHEDULE"] = old


def test_attention_workspace_covers_both_schedules(lib):
    """The workspace holds the partial storage of either work schedule, so its
    size does not depend on DP_ATTN_SCHEDULE: S key chunks of float32 rows
    plus (reference, sum) pairs for a split, two 128-row pieces per resident
    block (a multiple of 8 blocks, whatever the shape) for the balanced
    schedule."""
    piece = 2 * (128 * 64 + 128 * 2) * 4
    shapes = ((1, 1, 128, 64), (2, 10, 7200, 57600), (1, 4, 300, 2049), (2, 10, 1024, 4096))
    for shp in shapes:
        sizes = {_attn_ws(lib, s, *shp) for s in (None, "split", "balanced", "bogus")}
        assert len(sizes) == 1, (shp, sizes)
        ws = sizes.pop()
        assert ws > 0 and ws >= 8 * piece
    # a single unsplit round needs only the balanced pieces
    small = _attn_ws(lib, None, 1, 1, 128, 64)
    assert small % (8 * piece) == 0
    # the SDXL-3840 share's split keeps at least two key chunks of partials
    B, H, Tq = 2, 10, 7200
    per_chunk = B * Tq * H * 64 * 4 + B * H * Tq * 2 * 4
    assert _attn_ws(lib, None, B, H, Tq, 57600) >= 2 * per_chunk


def test_conv_and_linear_validation(lib):
    st, _ = status_and_error(lib.dp_conv3x3_stale_halo, A, None, None, Bp, None, Cp, 2, 4, 8, 48, 64,
                             _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_UNSUPPORTED
    st, _ = status_and_error(lib.dp_conv3x3_stale_halo, A, None, None, Bp, None, Cp, 2, 4, 8, 64, 40,
                             _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_UNSUPPORTED
    st, _ = status_and_error(lib.dp_conv3x3_stale_halo, None, None, None, Bp, None, Cp, 2, 4, 8, 64, 64,
                             _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    st, _ = status_and_error(lib.dp_conv3x3_stale_halo, A, None, None, Bp, None, Cp, 2, 0, 8, 64, 64,
                             _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    st, _ = status_and_error(lib.dp_linear, A, Bp, None, Cp, 100, 48, 64, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_UNSUPPORTED
    st, _ = status_and_error(lib.dp_linear, A, Bp, None, Cp, -1, 64, 64, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    st, msg = status_and_error(lib.dp_linear, A, Bp, None, A + 16, 100, 64, 64, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG and "overlap" in msg


def test_groupnorm_validation(lib):
    need = lib.dp_groupnorm_stale_stats_workspace(2, 7200, 640, 32)
    assert need > 0
    base = dict(x=A, stale=Bp, n=4, rank=1, T_total=4 * 7200, gamma=None, beta=None, eps=1e-5,
                silu=0, y=Cp, fresh=None, B=2, T=7200, C=640, G=32, dt=_lib.DP_BF16, ws=D, ws_bytes=need)

    def call(**kw):
        a = {**base, **kw}
        return status_and_error(lib.dp_groupnorm_stale_stats, a["x"], a["stale"], a["n"], a["rank"],
                                a["T_total"], a["gamma"], a["beta"], a["eps"], a["silu"], a["y"],
                                a["fresh"], a["B"], a["T"], a["C"], a["G"], a["dt"], a["ws"],
                                a["ws_bytes"], None)[0]

    assert call(rank=4) == _lib.DP_ERR_INVALID_ARG
    assert call(rank=-1) == _lib.DP_ERR_INVALID_ARG
    assert call(T_total=100) == _lib.DP_ERR_INVALID_ARG
    assert call(eps=-1.0) == _lib.DP_ERR_INVALID_ARG
    assert call(G=7) == _lib.DP_ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == _lib.DP_ERR_INVALID_ARG
    assert call(stale=None) == _lib.DP_ERR_INVALID_ARG
    need2 = lib.dp_groupnorm_stale_stats_workspace(2, 7200, 4096, 32)
    assert call(C=4096, ws_bytes=need2) == _lib.DP_ERR_UNSUPPORTED
    assert call(y=A + 2) == _lib.DP_ERR_INVALID_ARG


def test_qkv_projection_validation(lib):
    F, G2, H2 = 0x60000000, 0x70000000, 0x80000000
    f = lib.dp_qkv_projection_into_buffers
    # rows [t0, t0 + T_loc) must lie inside the buffer
    st, _ = status_and_error(f, A, Bp, Cp, D, E, F, G2, 2, 64, 256, 200, 64, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    st, _ = status_and_error(f, A, Bp, Cp, D, E, F, G2, 2, 64, 256, -1, 64, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    st, _ = status_and_error(f, A, Bp, Cp, None, E, F, G2, 2, 64, 256, 0, 64, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG
    # the two buffers may not overlap each other
    st, msg = status_and_error(f, A, Bp, Cp, D, E, F, F + 64, 2, 64, 256, 0, 64, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG and "overlap" in msg
    # bf16 needs C % 32 == 0
    st, _ = status_and_error(f, A, Bp, Cp, D, E, F, H2, 2, 64, 256, 0, 48, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_UNSUPPORTED


def test_otil_validation(lib):
    F2, G2 = 0x60000000, 0x70000000
    sp = lib.dp_otil_select_pack
    ok = (A, Bp, Cp, D, E, F2, 2, 32, 128, 4, 8, 8, 32, 10.0, _lib.DP_F16, None)

    def call(**kw):
        names = ["x", "last", "vis", "scores", "idx", "packed", "B", "h", "W", "C", "bh", "bw", "k",
                 "bonus", "dt", "st"]
        args = dict(zip(names, ok))
        args.update(kw)
        return status_and_error(sp, *[args[n] for n in names])

    assert call(x=None)[0] == _lib.DP_ERR_INVALID_ARG
    assert call(h=30)[0] == _lib.DP_ERR_INVALID_ARG            # 30 % 8 != 0
    assert call(k=65)[0] == _lib.DP_ERR_INVALID_ARG            # K = 4 * 16 = 64
    assert call(k=0)[0] == _lib.DP_ERR_INVALID_ARG
    assert call(bonus=float("inf"))[0] == _lib.DP_ERR_INVALID_ARG
    assert call(dt=7)[0] == _lib.DP_ERR_INVALID_ARG
    st, msg = call(packed=A + 64)
    assert st == _lib.DP_ERR_INVALID_ARG and "overlap" in msg
    assert call(x=A + 1)[0] == _lib.DP_ERR_INVALID_ARG          # misaligned f16 pointer
    assert call(h=256, W=512, bh=1, bw=1, k=1)[0] == _lib.DP_ERR_UNSUPPORTED  # K > 16384
    up = lib.dp_otil_unpack
    assert status_and_error(up, A, Bp, Cp, 2, 128, 128, 4, 100, 32, 8, 8, 32, _lib.DP_F16, None)[0] == \
        _lib.DP_ERR_INVALID_ARG                                  # rows [100, 132) outside H = 128
    assert status_and_error(up, A, Bp, None, 2, 128, 128, 4, 0, 32, 8, 8, 32, _lib.DP_F16, None)[0] == \
        _lib.DP_ERR_INVALID_ARG
    assert status_and_error(up, A, A + 128, G2, 2, 128, 128, 4, 0, 32, 8, 8, 32, _lib.DP_F16, None)[0] == \
        _lib.DP_ERR_INVALID_ARG                                  # dst overlaps packed
    # the other calls reject F16
    assert status_and_error(lib.dp_linear, A, Bp, None, Cp, 4, 32, 32, _lib.DP_F16, None)[0] == \
        _lib.DP_ERR_INVALID_ARG


def test_conv_gn_sums_and_apply_validation(lib):
    F2, G2 = 0x60000000, 0x70000000
    f = lib.dp_conv3x3_stale_halo_gn_sums
    need = lib.dp_conv3x3_gn_sums_workspace(2, 30, 240, 640)
    # partials for the smallest tile shape (64x64: 225 x 10 tiles) and one
    # channel per group (65 slots), two batch segments
    assert need >= 225 * 2 * 10 * 65 * 8
    ok = [A, None, None, Bp, None, Cp, D, 32, E, need, 2, 30, 240, 640, 640, _lib.DP_BF16, None]

    def call(i=None, v=None):
        a = list(ok)
        if i is not None:
            a[i] = v
        return status_and_error(f, *a)

    assert call(6, None)[0] == _lib.DP_ERR_INVALID_ARG              # NULL gn_sums
    assert call(7, 48)[0] == _lib.DP_ERR_INVALID_ARG                # Cout % G != 0
    assert call(9, need - 1)[0] == _lib.DP_ERR_INVALID_ARG          # short workspace
    assert call(15, _lib.DP_F32)[0] == _lib.DP_ERR_UNSUPPORTED       # bf16 only
    a = list(ok)
    a[11], a[12] = 1, 100                                           # h*W = 100 < 160
    a[9] = lib.dp_conv3x3_gn_sums_workspace(2, 1, 100, 640)
    assert status_and_error(f, *a)[0] == _lib.DP_ERR_UNSUPPORTED
    assert call(6, Cp + 64)[0] == _lib.DP_ERR_INVALID_ARG           # gn_sums inside y
    ap = lib.dp_groupnorm_apply
    st, _ = status_and_error(ap, A, None, F2, 4, 1, 1000, None, None, 1e-5, 0, G2, 2, 100, 64, 32,
                             _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG                             # NULL local sums
    st, _ = status_and_error(ap, A, Bp, F2, 4, 4, 1000, None, None, 1e-5, 0, G2, 2, 100, 64, 32,
                             _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG                             # rank outside [0, 4)


# Fake addresses 16 TB apart, so that the overlap checks pass for the huge
# sizes below and the size limits are what rejects each call.
FAR = [(i + 1) << 44 for i in range(8)]


def test_size_limits_are_rejected_before_launch(lib):
    """Every entry point refuses shapes beyond the 32-bit ranges its kernels
    index with (grid dimensions, buffer-descriptor byte counts, int rows)."""
    a, b, c, d, e, f, g, h = FAR
    bf = _lib.DP_BF16
    # attention: one batch item of K/V beyond 2^31 elements; more than 65535 heads
    st, msg = status_and_error(lib.dp_attn_stale_kv, a, b, c, d, 1, 10, 64, 4_000_000, 64, 0.0, bf,
                               None, 0, None)
    assert st == _lib.DP_ERR_UNSUPPORTED and "2^31" in msg
    st, _ = status_and_error(lib.dp_attn_stale_kv, a, b, c, d, 1, 70_000, 64, 64, 64, 0.0, bf, None, 0, None)
    assert st == _lib.DP_ERR_UNSUPPORTED
    # projection with 2^31 rows
    st, msg = status_and_error(lib.dp_linear, a, b, None, c, 1 << 31, 64, 64, bf, None)
    assert st == _lib.DP_ERR_UNSUPPORTED and "2^31" in msg
    # conv whose B*h*W reaches 2^32 rows
    st, msg = status_and_error(lib.dp_conv3x3_stale_halo, a, None, None, b, None, c, 2, 1 << 30, 2, 64, 64,
                               bf, None)
    assert st == _lib.DP_ERR_UNSUPPORTED and "2^31" in msg
    # fused Q/K/V projection into buffers of B*T_kv beyond 2^31 rows
    st, msg = status_and_error(lib.dp_qkv_projection_into_buffers, a, b, c, d, e, f, g, 2, 64, 1 << 30, 0, 64,
                               bf, None)
    assert st == _lib.DP_ERR_UNSUPPORTED and "2^31" in msg
    # GroupNorm over 2^31 local tokens (given a large enough workspace)
    need = lib.dp_groupnorm_stale_stats_workspace(1, 1 << 31, 64, 32)
    st, _ = status_and_error(lib.dp_groupnorm_stale_stats, a, None, 1, 0, 1 << 31, None, None, 1e-5, 0, b, None,
                             1, 1 << 31, 64, 32, bf, c, need, None)
    assert st == _lib.DP_ERR_UNSUPPORTED
    # splice with more (batch, K/V) segments than a grid dimension holds
    st, msg = status_and_error(lib.dp_kv_buffer_splice, a, b, c, d, 40_000, 16, 8, 0, 4, bf, None)
    assert st == _lib.DP_ERR_UNSUPPORTED and "grid" in msg


def test_groupnorm_noalloc_validation(lib):
    """The no-allocation GroupNorm rejects bad arguments, and shapes whose
    workspace exceeds its 4 MiB static scratch, before any HIP call."""
    def call(x=A, stale=Bp, n=4, rank=1, T_total=4 * 7200, y=Cp, B=2, T=7200, C=640, G=32):
        return status_and_error(lib.dp_groupnorm_stale_stats_noalloc, x, stale, n, rank, T_total, None, None,
                                1e-5, 0, y, None, B, T, C, G, _lib.DP_BF16, None)

    assert call(y=None)[0] == _lib.DP_ERR_INVALID_ARG
    assert call(rank=4)[0] == _lib.DP_ERR_INVALID_ARG
    assert call(G=7)[0] == _lib.DP_ERR_INVALID_ARG
    assert lib.dp_groupnorm_stale_stats_workspace(128, 4096, 2048, 2048) > 4 << 20
    st, msg = call(B=128, T=4096, C=2048, G=2048, T_total=4 * 4096)
    assert st == _lib.DP_ERR_UNSUPPORTED and "scratch" in msg
    # overlapping x and y: rejected before the first call's scratch set-up
    st, msg = call(y=A + 2)
    assert st == _lib.DP_ERR_INVALID_ARG and "overlap" in msg


def test_misaligned_vector_tensors_are_rejected(lib):
    """16-byte pieces: a bf16 tensor whose base is not 16-byte aligned is
    rejected on the host (the addresses are far apart: no overlap)."""
    st, msg = status_and_error(lib.dp_linear, A + 8, Bp, None, Cp, 64, 64, 64, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG and "aligned" in msg
    st, msg = status_and_error(lib.dp_linear, A, Bp, None, Cp + 2, 64, 64, 64, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG and "aligned" in msg
    st, msg = status_and_error(lib.dp_attn_stale_kv, A, Bp + 8, Cp, D, 1, 1, 64, 64, 64, 0.0, _lib.DP_BF16, E, 1 << 20,
                               None)
    assert st == _lib.DP_ERR_INVALID_ARG and "aligned" in msg
    st, msg = status_and_error(lib.dp_groupnorm_apply, A + 4, Bp, None, 1, 0, 64, None, None, 1e-5, 0, Cp, 1, 64, 64,
                               32, _lib.DP_BF16, None)
    assert st == _lib.DP_ERR_INVALID_ARG and "aligned" in msg
