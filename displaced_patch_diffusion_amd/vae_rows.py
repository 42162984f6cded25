"""Row-sharded VAE decoder resnet on one GPU (DistVAE row mode).

"Benchmarking DistVAE", "Default suite", item 2: adapted layers process
rank-local row bands, exchange halos and reassemble the output; "Glossary":
a halo is the neighbouring rows a sharded convolution needs.  Unlike the
displaced diffusion step, everything here is fresh: each conv takes its halo
rows from the neighbouring bands' current output, and each GroupNorm combines
the rank's own sums with the other bands' current sums (dp_groupnorm_sums).

One resnet = GN+SiLU -> conv3x3 -> GN+SiLU -> conv3x3.  In bf16 the first
conv also returns the GroupNorm sums of its output (its epilogue forms them),
so the second GroupNorm is a single pass.  Every step runs in libdp; this
module only orders the calls and slices the bands.
"""
from __future__ import annotations

import torch

from . import ops
from .partition import row_bands


class RowShardedResnet:
    """weights: torch tensors w0, w1 [C,3,3,C], b0, b1 [C] f32, gamma0/1, beta0/1 [C] f32."""

    def __init__(self, H: int, W: int, C: int, N: int, weights: dict, G: int = 32, eps: float = 1e-5):
        self.H, self.W, self.C, self.N, self.G, self.eps = H, W, C, N, G, eps
        self.wt = weights
        self.bands = row_bands(H, N)

    def _gn(self, xs: list, i: int, sums=None) -> list:
        """GroupNorm+SiLU of every band with whole-image statistics; `sums`
        [N,B,G,2] are the bands' own sums when a producer already formed them."""
        B = xs[0].shape[0]
        if sums is None:
            sums = torch.stack([ops.dp_groupnorm_sums(x.view(B, -1, self.C), self.G) for x in xs])
        out = []
        for r, x in enumerate(xs):
            # the band's own sums are sums[r]; the other bands' are the rest
            out.append(ops.dp_groupnorm_apply(
                x.view(B, -1, self.C), sums[r], sums, r, self.H * self.W, self.wt[f"gamma{i}"],
                self.wt[f"beta{i}"], self.eps, True, self.G).view_as(x))
        return out

    def _conv(self, ys: list, i: int, with_sums: bool = False):
        """conv3x3 of every band with fresh halo rows from its neighbours;
        with_sums also returns the bands' GroupNorm sums of the outputs
        [N,B,G,2], formed in the conv epilogue."""
        out, sums = [], []
        for r, y in enumerate(ys):
            top = ys[r - 1][:, -1].contiguous() if r > 0 else None
            bot = ys[r + 1][:, 0].contiguous() if r + 1 < self.N else None
            if with_sums:
                z, s = ops.dp_conv3x3_stale_halo_gn_sums(y, top, bot, self.wt[f"w{i}"], self.wt[f"b{i}"], self.G)
                out.append(z)
                sums.append(s)
            else:
                out.append(ops.dp_conv3x3_stale_halo(y, top, bot, self.wt[f"w{i}"], self.wt[f"b{i}"]))
        return (out, torch.stack(sums)) if with_sums else out

    def forward_bands(self, x_full: torch.Tensor) -> list:
        """x_full [B,H,W,C] -> the output bands [B,h_r,W,C]."""
        xs = [x_full[:, a:b].contiguous() for a, b in self.bands]
        if x_full.dtype != torch.bfloat16:  # the conv epilogue forms sums in bf16 only
            for i in range(2):
                xs = self._conv(self._gn(xs, i), i)
            return xs
        zs, sums = self._conv(self._gn(xs, 0), 0, with_sums=True)
        return self._conv(self._gn(zs, 1, sums), 1)

    def forward(self, x_full: torch.Tensor) -> torch.Tensor:
        return torch.cat(self.forward_bands(x_full), dim=1)
