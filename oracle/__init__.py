"""CPU oracle for one rank's share of a displaced-patch diffusion step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product path (the
HIP library and its Python binding) never does, and shares no code with it.

Arithmetic lives in ``dp_oracle.c`` (float64, plain loops, OpenMP over the
outermost independent index); this module marshals numpy arrays to it and
writes the two steps that are not arithmetic -- the row-band partition and
the K/V buffer splice -- directly in numpy.  All functions take and return
float64 arrays; callers widen bf16/fp32 storage values exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with the host compiler (gcc, OpenMP, -O2)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-fvisibility=hidden", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        D = ctypes.c_double
        lib.dpo_linear.argtypes = [P, P, P, P, I, I, I]
        lib.dpo_attention.argtypes = [P, P, P, P, I, I, I, I, I, D]
        lib.dpo_conv3x3_halo.argtypes = [P, P, P, P, P, P, I, I, I, I, I]
        lib.dpo_group_sums.argtypes = [P, I, I, I, I, P]
        lib.dpo_groupnorm_stale.argtypes = [P, P, I, I, I, P, P, D, ctypes.c_int, P, P, I, I, I, I]
        lib.dpo_partition_rows.argtypes = [I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
        for f in (lib.dpo_linear, lib.dpo_attention, lib.dpo_conv3x3_halo, lib.dpo_group_sums,
                  lib.dpo_groupnorm_stale, lib.dpo_partition_rows):
            f.restype = None
        _lib = lib
    return _lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ partition
def partition_rows(H: int, N: int, r: int) -> tuple[int, int]:
    """Rank r's row band [row0, row1) of an H-row image split over N ranks
    (DistVAE "Glossary": patchify into rank-local row bands)."""
    r0, r1 = ctypes.c_int64(), ctypes.c_int64()
    _load().dpo_partition_rows(H, N, r, ctypes.byref(r0), ctypes.byref(r1))
    return r0.value, r1.value


# --------------------------------------------------------------------- splice
def kv_buffer_splice(k_buf: np.ndarray, v_buf: np.ndarray, k_fresh: np.ndarray,
                     v_fresh: np.ndarray, t0: int) -> tuple[np.ndarray, np.ndarray]:
    """Copies of the [B,T_kv,C] buffers with tokens [t0, t0+T_loc) replaced by
    the fresh [B,T_loc,C] rows and every other token left as it was.  Works on
    any dtype, bit for bit ("OTIL ...", "Self-tests": the local slice comes out
    exactly fresh and a remote position is stale memory, never a blend)."""
    k_out, v_out = k_buf.copy(), v_buf.copy()
    T = k_fresh.shape[1]
    k_out[:, t0:t0 + T, :] = k_fresh
    v_out[:, t0:t0 + T, :] = v_fresh
    return k_out, v_out


# ----------------------------------------------------------------- arithmetic
def linear(x, w, bias=None):
    """y = x @ w.T (+ bias) over the last axis; x [..., Cin], w [Cout, Cin]."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    Cout, Cin = w.shape
    M = x.size // Cin
    y = np.empty(x.shape[:-1] + (Cout,), dtype=np.float64)
    _load().dpo_linear(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), M, Cin, Cout)
    return y


def attention(q, k, v, heads: int, scale: float | None = None):
    """q [B,Tq,C], k/v [B,Tkv,C] -> o [B,Tq,C]; scale None (or <= 0) = 1/sqrt(d)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Tq, C = q.shape
    Tkv = k.shape[1]
    d = C // heads
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    o = np.empty_like(q)
    _load().dpo_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, heads, Tq, Tkv, d, float(scale))
    return o


def conv3x3_halo(x, halo_top, halo_bot, w, bias=None):
    """x [B,h,W,Cin], halos [B,W,Cin] or None, w [Cout,3,3,Cin] -> y [B,h,W,Cout]."""
    x, ht, hb, w, bias = _f64(x), _f64(halo_top), _f64(halo_bot), _f64(w), _f64(bias)
    B, h, W, Cin = x.shape
    Cout = w.shape[0]
    y = np.empty((B, h, W, Cout), dtype=np.float64)
    _load().dpo_conv3x3_halo(_ptr(x), _ptr(ht), _ptr(hb), _ptr(w), _ptr(bias), _ptr(y),
                             B, h, W, Cin, Cout)
    return y


def group_sums(x, G: int):
    """x [B,T,C] -> [B,G,2] float64 (sum, sum of squares) per group."""
    x = _f64(x)
    B, T, C = x.shape
    s = np.empty((B, G, 2), dtype=np.float64)
    _load().dpo_group_sums(_ptr(x), B, T, C, G, _ptr(s))
    return s


def groupnorm_stale(x, stale_sums, rank: int, T_total: int, gamma=None, beta=None,
                    eps: float = 1e-5, silu: bool = False, G: int = 32):
    """x [B,T,C], stale_sums [N,B,G,2] -> (y [B,T,C], fresh local sums [B,G,2])."""
    x, st, gamma, beta = _f64(x), _f64(stale_sums), _f64(gamma), _f64(beta)
    B, T, C = x.shape
    N = st.shape[0]
    y = np.empty_like(x)
    fresh = np.empty((B, G, 2), dtype=np.float64)
    _load().dpo_groupnorm_stale(_ptr(x), _ptr(st), N, rank, T_total, _ptr(gamma), _ptr(beta),
                                float(eps), int(bool(silu)), _ptr(y), _ptr(fresh), B, T, C, G)
    return y, fresh


# ---------------------------------------------------------------------- chains
def attention_block_share(x_loc, wq, wk, wv, wo, k_buf, v_buf, t0: int, heads: int):
    """Projections of the local rows, splice of the fresh K/V into the
    full-image buffers, attention over all keys, output projection.
    Returns (y, k_spliced, v_spliced)."""
    q = linear(x_loc, wq)
    kf = linear(x_loc, wk)
    vf = linear(x_loc, wv)
    k_s, v_s = kv_buffer_splice(_f64(k_buf), _f64(v_buf), kf, vf, t0)
    o = attention(q, k_s, v_s, heads)
    return linear(o, wo), k_s, v_s


def rank_share_step(x_loc, wq, wk, wv, wo, k_buf, v_buf, t0, heads, W,
                    halo_top, halo_bot, conv_w, conv_b, stale_sums, rank, T_total,
                    gamma, beta, eps=1e-5, G=32):
    """Attention block -> conv3x3 with stale halos -> GroupNorm with stale sums,
    on one rank's rows.  x_loc [B,Tq,C]; returns a dict of every stage."""
    B, Tq, C = x_loc.shape
    y, k_s, v_s = attention_block_share(x_loc, wq, wk, wv, wo, k_buf, v_buf, t0, heads)
    h = Tq // W
    z = conv3x3_halo(y.reshape(B, h, W, C), halo_top, halo_bot, conv_w, conv_b)
    out, fresh = groupnorm_stale(z.reshape(B, Tq, -1), stale_sums, rank, T_total, gamma, beta,
                                 eps, False, G)
    return {"attn_out": y, "k_spliced": k_s, "v_spliced": v_s, "conv_out": z.reshape(B, Tq, -1),
            "out": out, "fresh_sums": fresh}


class DisplacedSchedule:
    """Several denoising steps of one layer stack -- attention block, 3x3
    conv, GroupNorm -- over N row bands, each step feeding its output to the
    next ("DistriFusion" project summary, "How It Works": a synchronous step,
    then steps that reuse the activations the other devices produced one step
    earlier; "OTIL for SDXL on 4x L40S", "What is implemented where": the
    stale state is the K/V buffers, the conv halo rows and two GroupNorm
    scalars per group).

    A synchronous step gives every band the current step's K/V rows, halo
    rows and group sums of all bands (the unsplit computation).  A displaced
    step gives band r its own fresh values and, for every other band, the
    values recorded during the previous step.  Every step records its full
    K/V buffers, each band's attention-block output rows and each band's
    fresh group sums.

    ``store(a)`` is applied wherever the device path stores a tensor (q, k,
    v, attention output, block output, conv output, step output), and
    ``store_sums`` to the recorded group sums (float32 on the device), so
    that the oracle sees the same rounded operands.
    """

    def __init__(self, H, W, heads, N, weights, G=32, eps=1e-5, store=None, store_sums=None):
        self.H, self.W, self.heads, self.N, self.G, self.eps = H, W, heads, N, G, eps
        self.wt = {k: _f64(v) if v is not None else None for k, v in weights.items()}
        self.store = store or (lambda a: a)
        self.store_sums = store_sums or (lambda a: a)
        self.bands = [partition_rows(H, N, r) for r in range(N)]
        self.prev = None

    def step(self, x, sync: bool, alpha: float = 1.0):
        """x [B, H*W, C] -> x + alpha (stack(x) - x), the synthetic sampler
        update between steps (alpha = 1: the stack's output); records this
        step's state."""
        if not sync and self.prev is None:
            raise ValueError("a displaced step needs a previous step")
        x = _f64(x)
        W, wt, s = self.W, self.wt, self.store
        B, T, C = x.shape
        band_x = [x[:, r0 * W:r1 * W] for r0, r1 in self.bands]
        q = [s(linear(xb, wt["wq"])) for xb in band_x]
        kf = [s(linear(xb, wt["wk"])) for xb in band_x]
        vf = [s(linear(xb, wt["wv"])) for xb in band_x]
        k_now, v_now = np.concatenate(kf, 1), np.concatenate(vf, 1)
        ys = []
        for r, (r0, r1) in enumerate(self.bands):
            if sync:
                kb, vb = k_now, v_now
            else:
                kb, vb = kv_buffer_splice(self.prev["k"], self.prev["v"], kf[r], vf[r], r0 * W)
            o = s(attention(q[r], kb, vb, self.heads))
            ys.append(s(linear(o, wt["wo"])))
        y_src = ys if sync else self.prev["y"]
        zs = []
        for r, (r0, r1) in enumerate(self.bands):
            h = r1 - r0
            top = y_src[r - 1].reshape(B, -1, W, C)[:, -1] if r0 > 0 else None
            bot = y_src[r + 1].reshape(B, -1, W, C)[:, 0] if r1 < self.H else None
            z = conv3x3_halo(ys[r].reshape(B, h, W, C), top, bot, wt["conv_w"], wt["conv_b"])
            zs.append(s(z.reshape(B, h * W, -1)))
        sums_now = np.stack([self.store_sums(group_sums(z, self.G)) for z in zs])
        stale = sums_now if sync else self.prev["sums"]
        outs = []
        for r in range(self.N):
            out, _ = groupnorm_stale(zs[r], stale, r, T, wt["gamma"], wt["beta"], self.eps, False, self.G)
            outs.append(s(out))
        self.prev = {"k": k_now, "v": v_now, "y": ys, "sums": sums_now}
        out = np.concatenate(outs, 1)
        return out if alpha == 1.0 else s(x + alpha * (out - x))
