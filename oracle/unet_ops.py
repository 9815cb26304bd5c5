"""CPU double-precision oracle for the UNet's group normalisation and its
GELU-gated product (the two other specialised kernels of the method).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``, never by the product package.  It
shares no code with the HIP library; the C source it wraps is ``unet_ops.c`` in
this directory (plain C99, double precision).

Method: "Speed Is All You Need: On-Device Acceleration of Large Diffusion
Models via GPU-Aware Optimizations" (Chen et al.), news write-up, section on
the specialised kernels (group normalisation over channel groups; GELU with the
Gaussian error function, fused with the split and the multiplication around
it).  The readings of what the pages leave open are stated in unet_ops.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "unet_ops.c")
_LIB = os.path.join(_HERE, "liboracle_ops.so")
# Test hook: the mutation tests point this at a deliberately broken build.
_LIB_OVERRIDE = os.environ.get("ATTN_ORACLE_OPS_LIB")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile unet_ops.c into liboracle_ops.so next to it (gcc, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(_LIB_OVERRIDE if _LIB_OVERRIDE else build())
        lib.oracle_group_norm.argtypes = [_D, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_double, _D, _D, _D]
        lib.oracle_group_norm.restype = ctypes.c_int
        lib.oracle_gelu1.argtypes = [ctypes.c_double]
        lib.oracle_gelu1.restype = ctypes.c_double
        lib.oracle_gelu.argtypes = [_D, ctypes.c_size_t, _D]
        lib.oracle_gelu.restype = None
        lib.oracle_geglu.argtypes = [_D, ctypes.c_int, ctypes.c_int, _D]
        lib.oracle_geglu.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _dp(a):
    return None if a is None else a.ctypes.data_as(_D)


def group_norm(x, groups: int, gamma=None, beta=None, eps: float = 1e-5):
    """Group normalisation of x [N, C, *spatial] -> (y, mean [N, G], rstd [N, G])."""
    x = _f64(x)
    n, c = x.shape[:2]
    hw = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
    ga = None if gamma is None else _f64(gamma)
    be = None if beta is None else _f64(beta)
    assert ga is None or ga.shape == (c,)
    assert be is None or be.shape == (c,)
    y = np.empty_like(x)
    mean = np.empty((n, groups), np.float64)
    rstd = np.empty((n, groups), np.float64)
    rc = _load().oracle_group_norm(_dp(x), _dp(ga), _dp(be), n, c, hw, int(groups), float(eps),
                                   _dp(y), _dp(mean), _dp(rstd))
    if rc != 0:
        raise ValueError(f"oracle_group_norm rejected N={n} C={c} HW={hw} groups={groups} eps={eps}")
    return y, mean, rstd


def gelu(x) -> np.ndarray:
    """x * Phi(x), element-wise."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().oracle_gelu(_dp(x), x.size, _dp(y))
    return y


def gelu1(x: float) -> float:
    return float(_load().oracle_gelu1(float(x)))


def geglu(h) -> np.ndarray:
    """h [..., 2F] -> h[..., :F] * gelu(h[..., F:])."""
    h = _f64(h)
    f2 = h.shape[-1]
    assert f2 % 2 == 0
    rows = int(np.prod(h.shape[:-1])) if h.ndim > 1 else 1
    out = np.empty(h.shape[:-1] + (f2 // 2,), np.float64)
    rc = _load().oracle_geglu(_dp(h), rows, f2 // 2, _dp(out))
    if rc != 0:
        raise ValueError("oracle_geglu rejected the sizes")
    return out
