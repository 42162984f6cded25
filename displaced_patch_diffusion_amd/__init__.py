"""MI355X (gfx950) library for one rank's share of a displaced-patch diffusion step.

The compute lives in libdp.so (hand-written HIP kernels behind a C ABI,
declared in include/dp.h); this package is its thin Python binding.
"""
from ._lib import DPError, LIB_PATH  # noqa: F401
from .ops import (  # noqa: F401
    dp_attn_stale_kv,
    dp_attn_stale_kv_workspace,
    dp_conv3x3_stale_halo,
    dp_groupnorm_stale_stats,
    dp_groupnorm_stale_stats_workspace,
    dp_kv_buffer_splice,
    dp_linear,
)
