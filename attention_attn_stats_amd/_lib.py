"""ctypes view of libattn.so (the C ABI declared in include/attn.h).

The library is loaded from this package directory only; a missing library is
an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
F32, F16, BF16 = 0, 1, 2
AUTO, PARTIAL_FUSED, FLASH = 0, 1, 2

EXPORTS = ("attn_stats", "attn_pv", "attn_flash", "attn_forward", "attn_select",
           "attn_default_variant", "attn_select_reset", "attn_status_string",
           "attn_scores", "attn_scores_stats", "attn_scores_pv",
           "attn_stats_strided", "attn_pv_strided", "attn_flash_strided", "attn_forward_strided",
           "attn_group_norm", "attn_group_norm_workspace_size", "attn_geglu",
           "attn_group_norm_static")

_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


class Strides(ctypes.Structure):
    """attn_strides: element strides of a [B, H, N, d] tensor."""
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong), ("row", ctypes.c_longlong)]


class Layout(ctypes.Structure):
    """attn_layout: the strides of q, k, v and out."""
    _fields_ = [("q", Strides), ("k", Strides), ("v", Strides), ("out", Strides)]


_lp = ctypes.POINTER(Layout)


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Load libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m attention_attn_stats_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.attn_stats.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
    lib.attn_stats.restype = _i
    lib.attn_pv.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
    lib.attn_pv.restype = _i
    lib.attn_flash.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
    lib.attn_flash.restype = _i
    lib.attn_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.attn_forward.restype = _i
    lib.attn_select.argtypes = [_i, _i, _i, _i, _i, _i, _vp]
    lib.attn_select.restype = _i
    lib.attn_default_variant.argtypes = [_i]
    lib.attn_default_variant.restype = _i
    lib.attn_select_reset.argtypes = []
    lib.attn_select_reset.restype = None
    lib.attn_scores.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
    lib.attn_scores.restype = _i
    lib.attn_scores_stats.argtypes = [_vp, _vp, _i, _i, _i, _i, _vp]
    lib.attn_scores_stats.restype = _i
    lib.attn_scores_pv.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
    lib.attn_scores_pv.restype = _i
    lib.attn_stats_strided.argtypes = [_vp, _vp, _vp, _lp, _i, _i, _i, _i, _i, _f, _i, _vp]
    lib.attn_stats_strided.restype = _i
    lib.attn_pv_strided.argtypes = [_vp, _vp, _vp, _vp, _vp, _lp, _i, _i, _i, _i, _i, _f, _i, _vp]
    lib.attn_pv_strided.restype = _i
    lib.attn_flash_strided.argtypes = [_vp, _vp, _vp, _vp, _vp, _lp, _i, _i, _i, _i, _i, _f, _i, _vp]
    lib.attn_flash_strided.restype = _i
    lib.attn_forward_strided.argtypes = [_vp, _vp, _vp, _vp, _vp, _lp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.attn_forward_strided.restype = _i
    lib.attn_group_norm.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _i, _i, _i, _i, _f, _i, _vp]
    lib.attn_group_norm.restype = _i
    lib.attn_group_norm_static.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]
    lib.attn_group_norm_static.restype = _i
    lib.attn_group_norm_workspace_size.argtypes = [_vp, _vp, _i, _i, _i, _i, _i]
    lib.attn_group_norm_workspace_size.restype = ctypes.c_size_t
    lib.attn_geglu.argtypes = [_vp, _vp, _i, _i, _i, _vp]
    lib.attn_geglu.restype = _i
    lib.attn_status_string.argtypes = [_i]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()
