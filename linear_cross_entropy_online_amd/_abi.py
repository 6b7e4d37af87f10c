"""ctypes view of include/flce.h: constants, structs, prototypes, library loader."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libflce.so")

FLCE_OK, FLCE_E_NULL, FLCE_E_SHAPE, FLCE_E_DTYPE, FLCE_E_ALIGN = 0, 1, 2, 3, 4
FLCE_E_WORKSPACE, FLCE_E_UNSUPPORTED, FLCE_E_LAUNCH, FLCE_E_DEVICE = 5, 6, 7, 8
FLCE_BF16, FLCE_F32 = 0, 1
FLCE_MEAN, FLCE_SUM, FLCE_NONE = 0, 1, 2
FLCE_FLAG_PROFILE = 1
FLCE_FLAG_COMPACT_IGNORED = 2
FLCE_FLAG_BF16_GRADS = 4
FLCE_FLAG_FILTER_FULL_C = 8
FLCE_FLAG_FILTER_FULL_E = 16
FLCE_FLAG_SORT_VOCAB = 32
FLCE_FLAG_WIDE_GRAD_TILES = 64
(FLCE_K_FWD_LSE, FLCE_K_LSE_COMBINE, FLCE_K_FINALIZE, FLCE_K_BWD_DZ, FLCE_K_BWD_GRAD,
 FLCE_K_AUX, FLCE_K_BWD_BAND, FLCE_K_COUNT) = range(8)

# Every function include/flce.h declares (checked against the header by a CPU test).
EXPORTS = ["flce_workspace_bytes", "flce_plan", "flce_forward", "flce_backward",
           "flce_fused_fwd_bwd", "flce_fused_fwd_bwd_noalloc",
           "flce_fused_fwd_bwd_kahan", "flce_backward_kahan", "flce_scale_gradients", "flce_filter_stats", "flce_device_status",
           "flce_strerror",
           "flce_profile_reset", "flce_profile_read", "flce_version"]


class FlceDesc(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("hidden", ctypes.c_int64), ("vocab", ctypes.c_int64),
                ("in_dtype", ctypes.c_int32), ("reduction", ctypes.c_int32),
                ("ignore_index", ctypes.c_int64), ("filter_eps", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("ws_budget_bytes", ctypes.c_uint64)]


class FlcePlanInfo(ctypes.Structure):
    _fields_ = [("ws_bytes", ctypes.c_int64), ("band_rows", ctypes.c_int32),
                ("band_vocab", ctypes.c_int32), ("n_bands_rows", ctypes.c_int32),
                ("n_bands_vocab", ctypes.c_int32), ("fwd_band_rows", ctypes.c_int32),
                ("fwd_workgroups", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("filter_block", ctypes.c_int32), ("dz_bytes", ctypes.c_int64),
                ("vocab_order_offset", ctypes.c_int64), ("grad_tile_d", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class FlceError(RuntimeError):
    def __init__(self, code: int, msg: str | None = None):
        self.code = code
        super().__init__(f"flce error {code}: {msg or strerror(code)}")


_LIB = None


def lib():
    """Load libflce.so from the package directory (raises if it is not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m linear_cross_entropy_online_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
    pd = ctypes.POINTER(FlceDesc)
    L.flce_workspace_bytes.argtypes = [pd]
    L.flce_workspace_bytes.restype = sz
    L.flce_plan.argtypes = [pd, ctypes.POINTER(FlcePlanInfo)]
    L.flce_plan.restype = i32
    L.flce_forward.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.flce_forward.restype = i32
    L.flce_backward.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.flce_backward.restype = i32
    L.flce_fused_fwd_bwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.flce_fused_fwd_bwd.restype = i32
    L.flce_fused_fwd_bwd_kahan.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.flce_fused_fwd_bwd_kahan.restype = i32
    L.flce_backward_kahan.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.flce_backward_kahan.restype = i32
    L.flce_fused_fwd_bwd_noalloc.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.flce_fused_fwd_bwd_noalloc.restype = i32
    L.flce_scale_gradients.argtypes = [pd, vp, vp, vp, vp]
    L.flce_scale_gradients.restype = i32
    L.flce_filter_stats.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int64)]
    L.flce_filter_stats.restype = i32
    L.flce_device_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32)]
    L.flce_device_status.restype = i32
    L.flce_strerror.argtypes = [i32]
    L.flce_strerror.restype = ctypes.c_char_p
    L.flce_profile_reset.argtypes = []
    L.flce_profile_reset.restype = i32
    L.flce_profile_read.argtypes = [i32, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]
    L.flce_profile_read.restype = i32
    L.flce_version.argtypes = []
    L.flce_version.restype = ctypes.c_char_p
    _LIB = L
    return L


def strerror(code: int) -> str:
    try:
        return lib().flce_strerror(int(code)).decode()
    except Exception:  # library unavailable while formatting an error
        return "error"


def check(rc: int):
    if rc != FLCE_OK:
        raise FlceError(rc)
