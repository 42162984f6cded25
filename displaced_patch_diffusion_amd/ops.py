"""Python binding of libdp: one function per C entry point, same names.

Argument marshalling only: tensors must already be contiguous device tensors
of the right dtype; every step runs in libdp's HIP kernels on torch's current
stream.  Outputs and workspaces are allocated here with torch when the caller
does not pass them.
"""
from __future__ import annotations

import torch

from ._lib import DP_BF16, DP_F16, DP_F32, check, lib

_DT = {torch.bfloat16: DP_BF16, torch.float32: DP_F32}


def _dt(*ts) -> int:
    dts = {t.dtype for t in ts if t is not None}
    if len(dts) != 1 or next(iter(dts)) not in _DT:
        raise TypeError(f"expected one of bf16/f32 for all tensors, got {dts}")
    return _DT[dts.pop()]


def _dev(*ts, f32=()):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous and on the GPU")
    for t in f32:
        if t is not None and (t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError("statistics, gamma/beta and bias must be contiguous float32 GPU tensors")


def _p(t):
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ws(nbytes: int, device) -> torch.Tensor | None:
    # zero-filled: the GroupNorm workspaces hold ticket counters that must
    # start at zero (every call leaves them at zero again)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def dp_kv_buffer_splice(k_buf, v_buf, k_fresh, v_fresh, t0: int) -> None:
    """In place: k_buf/v_buf [B,T_kv,C] tokens [t0, t0+T_loc) <- k_fresh/v_fresh [B,T_loc,C]."""
    _dev(k_buf, v_buf, k_fresh, v_fresh)
    dt = _dt(k_buf, v_buf, k_fresh, v_fresh)
    B, T_kv, C = k_buf.shape
    if tuple(v_buf.shape) != (B, T_kv, C) or k_fresh.shape != v_fresh.shape or \
            k_fresh.shape[0] != B or k_fresh.shape[2] != C:
        raise ValueError("shape mismatch")
    check(lib().dp_kv_buffer_splice(_p(k_buf), _p(v_buf), _p(k_fresh), _p(v_fresh), B, T_kv, C,
                                    t0, k_fresh.shape[1], dt, _stream()), "dp_kv_buffer_splice")


def dp_attn_stale_kv_workspace(B, H, Tq, T_kv, d, dtype) -> int:
    return lib().dp_attn_stale_kv_workspace(B, H, Tq, T_kv, d, _DT[dtype])


def dp_attn_stale_kv(q, k_buf, v_buf, heads: int, scale: float = 0.0, out=None, ws=None):
    """q [B,Tq,C], k_buf/v_buf [B,T_kv,C] -> out [B,Tq,C]; scale <= 0 means 1/sqrt(d)."""
    _dev(q, k_buf, v_buf, out)
    dt = _dt(q, k_buf, v_buf, out)
    B, Tq, C = q.shape
    T_kv = k_buf.shape[1]
    if tuple(k_buf.shape) != (B, T_kv, C) or tuple(v_buf.shape) != (B, T_kv, C) or C % heads:
        raise ValueError("shape mismatch")
    d = C // heads
    if out is None:
        out = torch.empty_like(q)
    need = lib().dp_attn_stale_kv_workspace(B, heads, Tq, T_kv, d, dt)
    if ws is None:
        ws = _ws(need, q.device)
    check(lib().dp_attn_stale_kv(_p(q), _p(k_buf), _p(v_buf), _p(out), B, heads, Tq, T_kv, d,
                                 float(scale), dt, _p(ws), 0 if ws is None else ws.numel(),
                                 _stream()), "dp_attn_stale_kv")
    return out


def dp_conv3x3_stale_halo(x, halo_top, halo_bot, w, bias=None, y=None):
    """x [B,h,W,Cin], halos [B,W,Cin] or None, w [Cout,3,3,Cin] -> y [B,h,W,Cout]."""
    _dev(x, halo_top, halo_bot, w, y, f32=(bias,))
    dt = _dt(x, halo_top, halo_bot, w, y)
    B, h, W, Cin = x.shape
    Cout = w.shape[0]
    if tuple(w.shape) != (Cout, 3, 3, Cin):
        raise ValueError("w must be [Cout,3,3,Cin]")
    for hl in (halo_top, halo_bot):
        if hl is not None and tuple(hl.shape) != (B, W, Cin):
            raise ValueError("halo must be [B,W,Cin]")
    if y is None:
        y = torch.empty((B, h, W, Cout), dtype=x.dtype, device=x.device)
    check(lib().dp_conv3x3_stale_halo(_p(x), _p(halo_top), _p(halo_bot), _p(w), _p(bias), _p(y),
                                      B, h, W, Cin, Cout, dt, _stream()), "dp_conv3x3_stale_halo")
    return y


def dp_groupnorm_stale_stats_workspace(B, T_loc, C, G) -> int:
    return lib().dp_groupnorm_stale_stats_workspace(B, T_loc, C, G)


def dp_groupnorm_stale_stats(x, stale_sums, rank: int, T_total: int, gamma=None, beta=None,
                             eps: float = 1e-5, fuse_silu: bool = False, G: int = 32, y=None,
                             fresh_sums_out=None, ws=None):
    """x [B,T_loc,C], stale_sums [N,B,G,2] f32 -> y [B,T_loc,C] (fresh sums into fresh_sums_out)."""
    _dev(x, y, f32=(stale_sums, gamma, beta, fresh_sums_out))
    dt = _dt(x, y)
    B, T, C = x.shape
    n_patches = 1 if stale_sums is None else stale_sums.shape[0]
    if stale_sums is not None and tuple(stale_sums.shape) != (n_patches, B, G, 2):
        raise ValueError("stale_sums must be [N,B,G,2]")
    if y is None:
        y = torch.empty_like(x)
    need = lib().dp_groupnorm_stale_stats_workspace(B, T, C, G)
    if ws is None:
        ws = _ws(need, x.device)
    check(lib().dp_groupnorm_stale_stats(_p(x), _p(stale_sums), n_patches, rank, T_total, _p(gamma),
                                         _p(beta), float(eps), int(bool(fuse_silu)), _p(y),
                                         _p(fresh_sums_out), B, T, C, G, dt, _p(ws),
                                         0 if ws is None else ws.numel(), _stream()),
          "dp_groupnorm_stale_stats")
    return y


def dp_groupnorm_stale_stats_noalloc(x, stale_sums, rank: int, T_total: int, gamma, beta, eps: float,
                                     fuse_silu: bool, G: int, y, fresh_sums_out=None):
    """dp_groupnorm_stale_stats with the library's static device scratch as
    its workspace: the call allocates nothing (y is the caller's)."""
    _dev(x, y, f32=(stale_sums, gamma, beta, fresh_sums_out))
    dt = _dt(x, y)
    B, T, C = x.shape
    n_patches = 1 if stale_sums is None else stale_sums.shape[0]
    if stale_sums is not None and tuple(stale_sums.shape) != (n_patches, B, G, 2):
        raise ValueError("stale_sums must be [N,B,G,2]")
    check(lib().dp_groupnorm_stale_stats_noalloc(_p(x), _p(stale_sums), n_patches, rank, T_total, _p(gamma),
                                                 _p(beta), float(eps), int(bool(fuse_silu)), _p(y),
                                                 _p(fresh_sums_out), B, T, C, G, dt, _stream()),
          "dp_groupnorm_stale_stats_noalloc")
    return y


def dp_groupnorm_sums(x, G: int = 32, out=None, ws=None):
    """x [B,T_loc,C] -> (sum x, sum x^2) per group, [B,G,2] float32."""
    _dev(x, out, ws)
    dt = _dt(x)
    B, T_loc, C = x.shape
    if out is None:
        out = torch.empty((B, G, 2), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = _ws(lib().dp_groupnorm_stale_stats_workspace(B, T_loc, C, G), x.device)
    check(lib().dp_groupnorm_sums(_p(x), _p(out), B, T_loc, C, G, dt, _p(ws),
                                  0 if ws is None else ws.numel(), _stream()), "dp_groupnorm_sums")
    return out


def dp_groupnorm_apply(x, local_sums, stale_sums, rank: int, T_total: int, gamma=None, beta=None,
                       eps: float = 1e-5, silu: bool = False, G: int = 32, y=None):
    """GroupNorm of x [B,T_loc,C] from the caller's local sums [B,G,2] plus the
    other patches' stale sums [N,B,G,2]."""
    _dev(x, y, f32=(local_sums, stale_sums, gamma, beta))
    dt = _dt(x, y)
    B, T_loc, C = x.shape
    n_patches = 1 if stale_sums is None else stale_sums.shape[0]
    if y is None:
        y = torch.empty_like(x)
    check(lib().dp_groupnorm_apply(_p(x), _p(local_sums), _p(stale_sums), n_patches, rank, T_total, _p(gamma),
                                   _p(beta), eps, int(silu), _p(y), B, T_loc, C, G, dt, _stream()),
          "dp_groupnorm_apply")
    return y


def dp_conv3x3_gn_sums_workspace(B, h, W, Cout) -> int:
    return lib().dp_conv3x3_gn_sums_workspace(B, h, W, Cout)


def dp_conv3x3_stale_halo_gn_sums(x, halo_top, halo_bot, w, bias=None, G: int = 32, y=None, gn_sums=None, ws=None):
    """conv3x3 of x [B,h,W,Cin] (as dp_conv3x3_stale_halo) plus the GroupNorm
    sums [B,G,2] of its output.  Returns (y, gn_sums)."""
    _dev(x, halo_top, halo_bot, w, y, ws, f32=(bias, gn_sums))
    dt = _dt(x, halo_top, halo_bot, w, y)
    B, h, W, Cin = x.shape
    Cout = w.shape[0]
    if tuple(w.shape) != (Cout, 3, 3, Cin):
        raise ValueError("w must be [Cout,3,3,Cin]")
    for hl in (halo_top, halo_bot):
        if hl is not None and tuple(hl.shape) != (B, W, Cin):
            raise ValueError("halo must be [B,W,Cin]")
    if y is None:
        y = torch.empty((B, h, W, Cout), dtype=x.dtype, device=x.device)
    if gn_sums is None:
        gn_sums = torch.empty((B, G, 2), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = _ws(dp_conv3x3_gn_sums_workspace(B, h, W, Cout), x.device)
    check(lib().dp_conv3x3_stale_halo_gn_sums(_p(x), _p(halo_top), _p(halo_bot), _p(w), _p(bias), _p(y),
                                              _p(gn_sums), G, _p(ws), 0 if ws is None else ws.numel(),
                                              B, h, W, Cin, Cout, dt, _stream()),
          "dp_conv3x3_stale_halo_gn_sums")
    return y, gn_sums


def dp_linear(x, w, bias=None, y=None):
    """x [..., Cin], w [Cout, Cin] -> y [..., Cout]."""
    _dev(x, w, y, f32=(bias,))
    dt = _dt(x, w, y)
    Cout, Cin = w.shape
    if x.shape[-1] != Cin:
        raise ValueError("x last dim must equal Cin")
    M = x.numel() // Cin
    if y is None:
        y = torch.empty(x.shape[:-1] + (Cout,), dtype=x.dtype, device=x.device)
    check(lib().dp_linear(_p(x), _p(w), _p(bias), _p(y), M, Cin, Cout, dt, _stream()), "dp_linear")
    return y


def dp_qkv_projection_into_buffers(x, wq, wk, wv, k_buf, v_buf, t0: int, q=None):
    """x [B,T_loc,C] -> q [B,T_loc,C]; K/V rows written into k_buf/v_buf [B,T_kv,C]
    at tokens [t0, t0+T_loc) (in place).  Returns q."""
    _dev(x, wq, wk, wv, k_buf, v_buf, q)
    dt = _dt(x, wq, wk, wv, k_buf, v_buf, q)
    B, T_loc, C = x.shape
    T_kv = k_buf.shape[1]
    if k_buf.shape != (B, T_kv, C) or v_buf.shape != k_buf.shape:
        raise ValueError("k_buf/v_buf must be [B,T_kv,C] with x's B and C")
    if any(w.shape != (C, C) for w in (wq, wk, wv)):
        raise ValueError("weights must be [C,C]")
    if q is None:
        q = torch.empty_like(x)
    check(lib().dp_qkv_projection_into_buffers(_p(x), _p(wq), _p(wk), _p(wv), _p(q), _p(k_buf),
                                               _p(v_buf), B, T_loc, T_kv, t0, C, dt, _stream()),
          "dp_qkv_projection_into_buffers")
    return q


_OTIL_DT = {torch.bfloat16: DP_BF16, torch.float32: DP_F32, torch.float16: DP_F16}


def dp_otil_select_pack(x, last_sent, visited, bh: int, bw: int, k: int, bonus: float = 10.0,
                        scores=None, idx=None, packed=None):
    """Sender side of OTIL for the band x [B,h,W,C]: updates last_sent and
    visited (uint8 [K]) in place; returns (scores [K] f32, idx [k] int32,
    packed [k,B,bh,bw,C])."""
    _dev(x, last_sent, visited, scores, idx, packed)
    if x.dtype not in _OTIL_DT or last_sent.dtype != x.dtype or (packed is not None and packed.dtype != x.dtype):
        raise TypeError("x, last_sent and packed must share one of f32/bf16/f16")
    if visited.dtype != torch.uint8:
        raise TypeError("visited must be uint8")
    B, h, W, C = x.shape
    if last_sent.shape != x.shape:
        raise ValueError("last_sent must have x's shape")
    K = (h // bh) * (W // bw) if bh > 0 and bw > 0 else 0
    if visited.numel() != K:
        raise ValueError(f"visited must hold {K} flags")
    if scores is None:
        scores = torch.empty(K, dtype=torch.float32, device=x.device)
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=x.device)
    if packed is None:
        packed = torch.empty((k, B, bh, bw, C), dtype=x.dtype, device=x.device)
    if scores.dtype != torch.float32 or idx.dtype != torch.int32:
        raise TypeError("scores must be float32 and idx int32")
    check(lib().dp_otil_select_pack(_p(x), _p(last_sent), _p(visited), _p(scores), _p(idx), _p(packed),
                                    B, h, W, C, bh, bw, k, bonus, _OTIL_DT[x.dtype], _stream()),
          "dp_otil_select_pack")
    return scores, idx, packed


def dp_otil_unpack(dst, packed, idx, r0: int, h: int, bh: int, bw: int) -> None:
    """Receiver side of OTIL: copies packed [k,B,bh,bw,C] blocks idx [k] into
    rows [r0, r0+h) of dst [B,H,W,C] (in place)."""
    _dev(dst, packed, idx)
    if dst.dtype not in _OTIL_DT or packed.dtype != dst.dtype or idx.dtype != torch.int32:
        raise TypeError("dst and packed must share one of f32/bf16/f16; idx must be int32")
    B, H, W, C = dst.shape
    k = idx.numel()
    if packed.shape != (k, B, bh, bw, C):
        raise ValueError("packed must be [k,B,bh,bw,C]")
    check(lib().dp_otil_unpack(_p(dst), _p(packed), _p(idx), B, H, W, C, r0, h, bh, bw, k,
                               _OTIL_DT[dst.dtype], _stream()), "dp_otil_unpack")
