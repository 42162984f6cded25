"""Row-band partition of a latent image over the ranks (the first step of a
rank's share).

Each rank owns a contiguous band of latent rows ("Benchmarking DistVAE",
"Glossary": patchify into rank-local row bands; "OTIL for SDXL on 4x L40S",
"Manual runs": a 2-way split has its seam at half the height).  With tokens
numbered row-major (t = row * W + col) a band is one contiguous token range,
which is what lets the attention buffers, the halo rows and the GroupNorm
bands of a share be plain pointer offsets.  Uneven splits take floors.
"""
from __future__ import annotations


def row_band(H: int, N: int, r: int) -> tuple[int, int]:
    """Rows [r0, r1) of rank r when H rows are split over N ranks."""
    if N <= 0 or not 0 <= r < N or H < 0:
        raise ValueError(f"row_band: need H >= 0 and 0 <= r < N, got H={H} N={N} r={r}")
    return (r * H) // N, ((r + 1) * H) // N


def row_bands(H: int, N: int) -> list[tuple[int, int]]:
    """Every rank's band, in rank order."""
    return [row_band(H, N, r) for r in range(N)]


def token_range(H: int, W: int, N: int, r: int) -> tuple[int, int]:
    """First token and token count of rank r's band (t0, T_loc)."""
    r0, r1 = row_band(H, N, r)
    return r0 * W, (r1 - r0) * W
