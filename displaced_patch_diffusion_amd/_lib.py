"""ctypes view of libdp.so: exported symbols and their C signatures.

Loading fails loudly when the library has not been built; there is no other
implementation behind these names.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdp.so")

P = ctypes.c_void_p
I64 = ctypes.c_int64
F32 = ctypes.c_float
SZ = ctypes.c_size_t
INT = ctypes.c_int

# name -> (restype, argtypes); the same list the header declares
SIGNATURES = {
    "dp_status_string": (ctypes.c_char_p, [INT]),
    "dp_last_error": (ctypes.c_char_p, []),
    "dp_kv_buffer_splice": (INT, [P, P, P, P, I64, I64, I64, I64, I64, INT, P]),
    "dp_attn_stale_kv_workspace": (SZ, [I64, I64, I64, I64, I64, INT]),
    "dp_attn_stale_kv": (INT, [P, P, P, P, I64, I64, I64, I64, I64, F32, INT, P, SZ, P]),
    "dp_conv3x3_stale_halo": (INT, [P, P, P, P, P, P, I64, I64, I64, I64, I64, INT, P]),
    "dp_groupnorm_stale_stats_workspace": (SZ, [I64, I64, I64, I64]),
    "dp_groupnorm_stale_stats": (INT, [P, P, I64, I64, I64, P, P, F32, INT, P, P, I64, I64, I64,
                                       I64, INT, P, SZ, P]),
    "dp_groupnorm_stale_stats_noalloc": (INT, [P, P, I64, I64, I64, P, P, F32, INT, P, P, I64, I64, I64,
                                               I64, INT, P]),
    "dp_groupnorm_sums": (INT, [P, P, I64, I64, I64, I64, INT, P, SZ, P]),
    "dp_groupnorm_apply": (INT, [P, P, P, I64, I64, I64, P, P, F32, INT, P, I64, I64, I64, I64, INT, P]),
    "dp_conv3x3_gn_sums_workspace": (SZ, [I64, I64, I64, I64]),
    "dp_conv3x3_stale_halo_gn_sums": (INT, [P, P, P, P, P, P, P, I64, P, SZ, I64, I64, I64, I64, I64, INT, P]),
    "dp_linear": (INT, [P, P, P, P, I64, I64, I64, INT, P]),
    "dp_qkv_projection_into_buffers": (INT, [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, INT, P]),
    "dp_otil_select_pack": (INT, [P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, I64, F32, INT, P]),
    "dp_otil_unpack": (INT, [P, P, P, I64, I64, I64, I64, I64, I64, I64, I64, I64, INT, P]),
}

DP_OK, DP_ERR_INVALID_ARG, DP_ERR_UNSUPPORTED, DP_ERR_HIP = 0, 1, 2, 3
DP_F32, DP_BF16, DP_F16 = 0, 1, 2

_lib = None


class DPError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: status {status} ({detail})")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m displaced_patch_diffusion_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(status: int, func: str) -> None:
    if status != DP_OK:
        detail = lib().dp_last_error().decode() or lib().dp_status_string(status).decode()
        raise DPError(status, func, detail)
