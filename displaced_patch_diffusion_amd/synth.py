"""Seeded synthetic inputs for one rank's share of a displaced-patch step.

This module draws random numbers and rounds them to the storage type, nothing
else: it holds none of the method's arithmetic (no projection, attention,
convolution or normalisation).  Both the CPU oracle (in the tests) and the HIP
path (tests and benchmark) take their inputs from here, so the two sides see
identical bits.

Each tensor comes from its own counter-free stream, seeded by
``(base seed, crc32(tensor name))``, so that adding or reordering draws never
changes another tensor.  Base seeds follow the seeded synthetic-weight
practice of the DistVAE benchmark README (opening paragraph): weights seed 0,
activations seed 1; stale-step noise uses seed 2 and affine/bias terms seed 3.

Shapes are those of SDXL-like UNet levels (the DistriFusion project summary,
"Highlighted Details", names SDXL up to 3840x3840); the image is split into
row bands, one per rank (DistVAE "Glossary": patchify).
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np

from .partition import row_band

SEED_WEIGHTS = 0
SEED_ACTIVATIONS = 1
SEED_STALE = 2
SEED_AFFINE = 3


# ---------------------------------------------------------------- bf16 storage
def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    a = np.array(a, dtype=np.float32, order="C", copy=True)
    if not np.isfinite(a).all():
        raise ValueError("round_to_bf16 expects finite values")
    u = a.reshape(-1).view(np.uint32)
    bias = np.empty(max(1, min(u.size, 1 << 20)), dtype=np.uint32)
    # finite floats are <= 0xFF7FFFFF, so adding at most 0x8000 cannot wrap
    for i in range(0, u.size, bias.size):
        seg = u[i:i + bias.size]
        b = bias[:seg.size]
        np.right_shift(seg, 16, out=b)
        b &= 1
        b += 0x7FFF
        seg += b
        seg &= 0xFFFF0000
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array whose values are representable in ``dtype`` ('f32'|'bf16'|'f16')."""
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f16":
        return np.asarray(a, np.float32).astype(np.float16).astype(np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    """One rank's share at one (or two) UNet levels.

    ``attn_*`` describe the self-attention level, ``conv_*`` the conv/GroupNorm
    level.  For the single-level workloads both are the same level and the
    chain is attention block -> conv3x3 -> GroupNorm.  For the two-level one
    the conv level runs GN+SiLU -> conv -> GN+SiLU -> conv and the attention
    level runs projections -> splice -> attention -> output projection.
    """

    name: str
    dtype: str
    B: int
    N: int
    rank: int
    attn_H: int
    attn_W: int
    attn_C: int
    heads: int
    head_dim: int
    conv_H: int
    conv_W: int
    conv_C: int
    two_level: bool = False
    G: int = 32
    eps: float = 1e-5
    noise: float = 0.05
    note: str = field(default="", compare=False)

    # attention level
    @property
    def T_kv(self) -> int:
        return self.attn_H * self.attn_W

    def rows(self, H: int, r: int | None = None) -> tuple[int, int]:
        return row_band(H, self.N, self.rank if r is None else r)

    def attn_rows(self, r: int | None = None) -> tuple[int, int]:
        return self.rows(self.attn_H, r)

    def conv_rows(self, r: int | None = None) -> tuple[int, int]:
        return self.rows(self.conv_H, r)

    @property
    def Tq(self) -> int:
        r0, r1 = self.attn_rows()
        return (r1 - r0) * self.attn_W

    @property
    def t0(self) -> int:
        return self.attn_rows()[0] * self.attn_W

    @property
    def conv_h(self) -> int:
        r0, r1 = self.conv_rows()
        return r1 - r0

    @property
    def conv_T(self) -> int:
        return self.conv_h * self.conv_W

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_rank(self, rank: int) -> "Workload":
        return Workload(**{**self.__dict__, "rank": rank})

    def with_noise(self, noise: float) -> "Workload":
        return Workload(**{**self.__dict__, "noise": noise})

    # algorithmic work of one step, counted as in the design notes
    def flops(self) -> dict:
        B, C, Ca = self.B, self.conv_C, self.attn_C
        attn = 4 * B * self.heads * self.Tq * self.T_kv * self.head_dim
        proj = 8 * B * self.Tq * Ca * Ca
        n_conv = 2 if self.two_level else 1
        conv = n_conv * 2 * B * self.conv_T * C * 9 * C
        return {"attn": attn, "proj": proj, "conv": conv}

    def bytes(self) -> dict:
        e = self.elem_bytes
        n_gn = 2 if self.two_level else 1
        gn = n_gn * 2 * self.B * self.conv_T * self.conv_C * e
        splice = 4 * self.B * self.Tq * self.attn_C * e
        return {"groupnorm": gn, "splice": splice}


def _single(name, dtype, H, W, C, heads, d, B, N, rank, note) -> Workload:
    return Workload(name=name, dtype=dtype, B=B, N=N, rank=rank, attn_H=H, attn_W=W,
                    attn_C=C, heads=heads, head_dim=d, conv_H=H, conv_W=W, conv_C=C,
                    note=note)


WORKLOADS: dict[str, Workload] = {
    "tiny32_c64_fp32": _single(
        "tiny32_c64_fp32", "f32", 32, 32, 64, 2, 32, 2, 2, 0,
        "latent 32x32, C=64, 2 heads x 32, batch 2, 2 row bands, rank 0"),
    "sdxl1024_l64_c640": _single(
        "sdxl1024_l64_c640", "bf16", 64, 64, 640, 10, 64, 2, 4, 1,
        "SDXL 1024^2, 64x64 level, C=640, 10x64 heads, batch 2, 4 row bands"),
    "sdxl1024_l32_c1280": _single(
        "sdxl1024_l32_c1280", "bf16", 32, 32, 1280, 20, 64, 2, 2, 1,
        "SDXL 1024^2, 32x32 level, C=1280, 20x64 heads, batch 2, 2 row bands"),
    "sdxl3840_l240_c640": _single(
        "sdxl3840_l240_c640", "bf16", 240, 240, 640, 10, 64, 2, 8, 1,
        "SDXL 3840^2, 240x240 level, C=640, 10x64 heads, batch 2, 8 row bands"),
    "sdxl2048_l256_c320_l128_c640": Workload(
        name="sdxl2048_l256_c320_l128_c640", dtype="bf16", B=2, N=4, rank=1,
        attn_H=128, attn_W=128, attn_C=640, heads=10, head_dim=64,
        conv_H=256, conv_W=256, conv_C=320, two_level=True,
        note="SDXL 2048^2: conv level 256x256 C=320 (GN+SiLU, conv, GN+SiLU, conv); "
             "attention level 128x128 C=640 10x64; batch 2, 4 row bands"),
}
WORKLOAD_ORDER = list(WORKLOADS)


# --------------------------------------------------------------------- drawing
_SALT = 0


def set_stream_salt(salt: int) -> None:
    """Select another family of streams (0, the default, is the one every
    test and stored value uses); the benchmark's --seed sets it."""
    global _SALT
    if salt < 0:
        raise ValueError("the salt must be >= 0")
    _SALT = int(salt)


def _rng(seed: int, name: str) -> np.random.Generator:
    key = [seed, zlib.crc32(name.encode())] + ([_SALT] if _SALT else [])
    return np.random.default_rng(np.random.SeedSequence(key))


def normal(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 N(mean, std^2) draws from the stream (seed, name)."""
    g = _rng(seed, name)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def attention_block_inputs(w: Workload, with_noise: bool = True) -> dict:
    """Full-image activations, the four projection weights and (unless
    with_noise is False) the stale-step noise for the attention level.  Stale
    K/V = (projection of the full image) + noise; the projection is left to
    the caller."""
    B, H, W, C, dt = w.B, w.attn_H, w.attn_W, w.attn_C, w.dtype
    s = 1.0 / np.sqrt(C)
    out = {
        "x_full": as_storage(normal(SEED_ACTIVATIONS, "attn.x_full", (B, H, W, C)), dt),
        "wq": as_storage(normal(SEED_WEIGHTS, "attn.wq", (C, C), s), dt),
        "wk": as_storage(normal(SEED_WEIGHTS, "attn.wk", (C, C), s), dt),
        "wv": as_storage(normal(SEED_WEIGHTS, "attn.wv", (C, C), s), dt),
        "wo": as_storage(normal(SEED_WEIGHTS, "attn.wo", (C, C), s), dt),
    }
    if with_noise:
        out["k_noise"] = normal(SEED_STALE, "attn.k_noise", (B, H * W, C), w.noise)
        out["v_noise"] = normal(SEED_STALE, "attn.v_noise", (B, H * W, C), w.noise)
    return out


def drawn_stale_state(w: Workload) -> dict:
    """A stale state drawn directly from the seeded streams, for parity runs
    whose expected values must not depend on a previous step computed on the
    device: remote K/V buffers ~ N(0,1) (the distribution of x W^T with
    x ~ N(0,1), W ~ N(0, 1/C)), halo rows ~ N(0,1) where the band has a
    neighbour, and the remote activations whose group sums stand for the other
    patches' stale sums (the sums themselves are arithmetic and are left to the
    caller).  Keys: k_buf, v_buf [B, T_kv, C]; halo_top{i}, halo_bot{i}
    [B, W, C] or None; remote{i} [N, B, T_band, C] for conv/GroupNorm layer i
    (the rank's own entry is drawn too and must never be read)."""
    B, C, dt = w.B, w.attn_C, w.dtype
    out = {
        "k_buf": as_storage(normal(SEED_STALE, "drawn.k_buf", (B, w.T_kv, C)), dt),
        "v_buf": as_storage(normal(SEED_STALE, "drawn.v_buf", (B, w.T_kv, C)), dt),
    }
    r0, r1 = w.conv_rows()
    Cc, Wc = w.conv_C, w.conv_W
    for i in range(2 if w.two_level else 1):
        out[f"halo_top{i}"] = (as_storage(normal(SEED_STALE, f"drawn.halo_top{i}", (B, Wc, Cc)), dt)
                               if r0 > 0 else None)
        out[f"halo_bot{i}"] = (as_storage(normal(SEED_STALE, f"drawn.halo_bot{i}", (B, Wc, Cc)), dt)
                               if r1 < w.conv_H else None)
        out[f"remote{i}"] = [
            as_storage(normal(SEED_STALE, f"drawn.remote{i}.{p}", (B, (w.conv_rows(p)[1] - w.conv_rows(p)[0]) * Wc, Cc),
                              1.1 + 0.1 * p, 0.05 * p), dt)
            for p in range(w.N)]
    return out


def conv_inputs(w: Workload, idx: int = 0) -> dict:
    """Conv weights [Cout,3,3,Cin] ~ N(0, 1/(9 Cin)), fp32 bias ~ N(0, 0.1^2),
    and stale-step noise for the two halo rows."""
    B, W, C, dt = w.B, w.conv_W, w.conv_C, w.dtype
    return {
        "w": as_storage(normal(SEED_WEIGHTS, f"conv{idx}.w", (C, 3, 3, C), 1.0 / np.sqrt(9 * C)), dt),
        "bias": normal(SEED_AFFINE, f"conv{idx}.bias", (C,), 0.1),
        "halo_top_noise": normal(SEED_STALE, f"conv{idx}.halo_top_noise", (B, W, C), w.noise),
        "halo_bot_noise": normal(SEED_STALE, f"conv{idx}.halo_bot_noise", (B, W, C), w.noise),
    }


def groupnorm_inputs(w: Workload, idx: int = 0) -> dict:
    """Per-channel fp32 affine terms: gamma ~ 1 + N(0, 0.1^2), beta ~ N(0, 0.1^2)."""
    C = w.conv_C
    return {
        "gamma": normal(SEED_AFFINE, f"gn{idx}.gamma", (C,), 0.1, 1.0),
        "beta": normal(SEED_AFFINE, f"gn{idx}.beta", (C,), 0.1),
    }


def conv_level_input(w: Workload, name: str = "conv.x_full") -> np.ndarray:
    """Full-image activations [B, H, W, C] ~ N(0,1) at the conv level."""
    return as_storage(normal(SEED_ACTIVATIONS, name, (w.B, w.conv_H, w.conv_W, w.conv_C)), w.dtype)


def stale_noise(w: Workload, name: str, shape) -> np.ndarray:
    return normal(SEED_STALE, name, shape, w.noise)


def random_tensor(seed: int, name: str, shape, dtype: str, std: float = 1.0) -> np.ndarray:
    return as_storage(normal(seed, name, shape, std), dtype)


def schedule_inputs(w: Workload) -> dict:
    """Initial full-image activations [B, H*W, C] and the weights of one layer
    stack (projections, conv, GroupNorm affine) for the multi-step schedule of
    a single-level workload; the same names and seeds as the per-op inputs."""
    if w.two_level:
        raise ValueError("the multi-step schedule runs single-level workloads")
    B, H, W, C, dt = w.B, w.attn_H, w.attn_W, w.attn_C, w.dtype
    s = 1.0 / np.sqrt(C)
    return {
        "x0": as_storage(normal(SEED_ACTIVATIONS, "attn.x_full", (B, H * W, C)), dt),
        "wq": as_storage(normal(SEED_WEIGHTS, "attn.wq", (C, C), s), dt),
        "wk": as_storage(normal(SEED_WEIGHTS, "attn.wk", (C, C), s), dt),
        "wv": as_storage(normal(SEED_WEIGHTS, "attn.wv", (C, C), s), dt),
        "wo": as_storage(normal(SEED_WEIGHTS, "attn.wo", (C, C), s), dt),
        "conv_w": as_storage(normal(SEED_WEIGHTS, "conv0.w", (C, 3, 3, C), 1.0 / np.sqrt(9 * C)), dt),
        "conv_b": normal(SEED_AFFINE, "conv0.bias", (C,), 0.1),
        "gamma": normal(SEED_AFFINE, "gn0.gamma", (C,), 0.1, 1.0),
        "beta": normal(SEED_AFFINE, "gn0.beta", (C,), 0.1),
    }


def otil_latent_sequence(seed: int, B: int, H: int, W: int, C: int, steps: int, bh: int, bw: int,
                         dtype: str) -> list:
    """A latent [B, H, W, C] over ``steps`` denoising steps, as a random walk in
    which each bh x bw block has its own step size: x_{s+1} = x_s + a_blk * N(0,1)
    with the block step sizes a distinct and spread over [0.02, 1] (so the
    blocks change by clearly different amounts).  Storage-rounded arrays."""
    nby, nbx = H // bh, W // bw
    amp = normal(seed, "otil.amp_order", (nby * nbx,))
    rank = np.argsort(np.argsort(amp))  # a random permutation of the block ids
    a = (0.02 + 0.98 * rank / max(nby * nbx - 1, 1)).astype(np.float32).reshape(nby, nbx)
    a_full = np.repeat(np.repeat(a, bh, axis=0), bw, axis=1)[None, :, :, None]
    x = normal(seed, "otil.x0", (B, H, W, C))
    out = [as_storage(x, dtype)]
    for s in range(1, steps):
        x = out[-1] + a_full * normal(seed, f"otil.step{s}", (B, H, W, C))
        out.append(as_storage(x, dtype))
    return out


# ------------------------------------------------------ row-sharded VAE decoder
@dataclass(frozen=True)
class VaeLevel:
    """One resnet of a KL-VAE decoder level, row-sharded over N ranks:
    GN+SiLU -> conv3x3 -> GN+SiLU -> conv3x3 on a [B, H, W, C] activation, with
    fresh halos and GroupNorm statistics over the whole image."""
    name: str
    dtype: str
    B: int
    H: int
    W: int
    C: int
    N: int
    rank: int
    G: int = 32
    eps: float = 1e-5
    note: str = field(default="", compare=False)

    def rows(self, r: int | None = None) -> tuple[int, int]:
        return row_band(self.H, self.N, self.rank if r is None else r)

    @property
    def h(self) -> int:
        r0, r1 = self.rows()
        return r1 - r0

    def conv_flops(self) -> int:
        """One conv of the rank's band (all nine taps counted)."""
        return 2 * self.B * self.h * self.W * self.C * 9 * self.C

    def gn_bytes(self) -> int:
        """One GroupNorm of the rank's band: read x, write y."""
        return 2 * self.B * self.h * self.W * self.C * (4 if self.dtype == "f32" else 2)


# The KL VAE decoder's widest levels at the pages' canonical sizes (the kl
# family's 1024x1024 and 2048x2048, 4 ranks): 128 channels at full resolution
# and 256 channels at half resolution.
VAE_LEVELS: dict[str, VaeLevel] = {
    "vae_kl1024_l1024_c128": VaeLevel("vae_kl1024_l1024_c128", "bf16", 1, 1024, 1024, 128, 4, 1,
                                      note="KL decoder, 1024^2 output, last level (128 ch), 4 ranks"),
    "vae_kl1024_l512_c256": VaeLevel("vae_kl1024_l512_c256", "bf16", 1, 512, 512, 256, 4, 1,
                                     note="KL decoder, 1024^2 output, 512^2 level (256 ch), 4 ranks"),
    "vae_kl2048_l2048_c128": VaeLevel("vae_kl2048_l2048_c128", "bf16", 1, 2048, 2048, 128, 4, 1,
                                      note="KL decoder, 2048^2 output, last level (128 ch), 4 ranks"),
    "vae_small_fp32": VaeLevel("vae_small_fp32", "f32", 2, 32, 24, 64, 4, 1,
                               note="small fp32 case the oracle runs in seconds"),
}


def vae_inputs(v: VaeLevel) -> dict:
    """Whole-image activation and the resnet's weights: weights seed 0,
    activation seed 1 (as the DistVAE bench builds its synthetic model)."""
    B, H, W, C, dt = v.B, v.H, v.W, v.C, v.dtype
    out = {"x": as_storage(normal(SEED_ACTIVATIONS, f"{v.name}.x", (B, H, W, C)), dt)}
    for i in range(2):
        out[f"w{i}"] = as_storage(normal(SEED_WEIGHTS, f"{v.name}.conv{i}.w", (C, 3, 3, C),
                                         1.0 / np.sqrt(9 * C)), dt)
        out[f"b{i}"] = normal(SEED_AFFINE, f"{v.name}.conv{i}.b", (C,), 0.1)
        out[f"gamma{i}"] = normal(SEED_AFFINE, f"{v.name}.gn{i}.gamma", (C,), 0.1, 1.0)
        out[f"beta{i}"] = normal(SEED_AFFINE, f"{v.name}.gn{i}.beta", (C,), 0.1)
    return out
