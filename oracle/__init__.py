"""CPU double-precision oracle for scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``, never by the product package.  It
shares no code with the HIP library; the C source it wraps is ``oracle.c`` in
this directory (plain C99, double precision, full score matrix materialised).

Method: "Speed Is All You Need: On-Device Acceleration of Large Diffusion
Models via GPU-Aware Optimizations" (Chen et al.), news write-up, section on
improving attention efficiency: the partially fused softmax reduces each row of
the logit matrix to a pair (m, l) and then fuses the softmax into the product
with V; FlashAttention is exact.  Both therefore equal the plain definition
computed here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Test hook: the mutation tests point this at a deliberately broken build of
# oracle.c to show that the pins catch it.
_LIB_OVERRIDE = os.environ.get("ATTN_ORACLE_LIB")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
             _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        lib.oracle_scores.argtypes = [_D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, _D]
        lib.oracle_scores.restype = None
        lib.oracle_softmax_rows.argtypes = [_D, ctypes.c_int, ctypes.c_int, _D, _D, _D]
        lib.oracle_softmax_rows.restype = None
        lib.oracle_pv.argtypes = [_D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int, _D]
        lib.oracle_pv.restype = None
        lib.oracle_block_stats.argtypes = [_D, ctypes.c_int, _I, ctypes.c_int, _D, _D]
        lib.oracle_block_stats.restype = None
        lib.oracle_attention.argtypes = [_D, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_double, _D, _D, ctypes.c_int]
        lib.oracle_attention.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dp(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def scores(q, k, scale: float) -> np.ndarray:
    """S = scale * q k^T for one head; q [nq, d], k [nk, d]."""
    q, k = _f64(q), _f64(k)
    nq, d = q.shape
    nk = k.shape[0]
    s = np.empty((nq, nk), np.float64)
    _load().oracle_scores(_dp(q), _dp(k), nq, nk, d, float(scale), _dp(s))
    return s


def softmax_rows(s):
    """Row softmax of S -> (P, m, l) with m the row max and l the sum of exp(s - m)."""
    s = _f64(s)
    nq, nk = s.shape
    p = np.empty_like(s)
    m = np.empty(nq, np.float64)
    l = np.empty(nq, np.float64)
    _load().oracle_softmax_rows(_dp(s), nq, nk, _dp(p), _dp(m), _dp(l))
    return p, m, l


def pv(p, v) -> np.ndarray:
    """O = P V for one head; p [nq, nk], v [nk, d]."""
    p, v = _f64(p), _f64(v)
    nq, nk = p.shape
    d = v.shape[1]
    o = np.empty((nq, d), np.float64)
    _load().oracle_pv(_dp(p), _dp(v), nq, nk, d, _dp(o))
    return o


def block_stats(row, block_lens):
    """(m, l) of one logit row via the block-split reduction with the given block lengths."""
    row = _f64(row)
    bl = np.ascontiguousarray(np.asarray(block_lens, dtype=np.int32))
    assert int(bl.sum()) == row.shape[0]
    m = ctypes.c_double()
    l = ctypes.c_double()
    _load().oracle_block_stats(_dp(row), row.shape[0], bl.ctypes.data_as(_I), bl.shape[0],
                               ctypes.byref(m), ctypes.byref(l))
    return m.value, l.value


def default_threads() -> int:
    """Threads of one oracle call: ATTN_ORACLE_THREADS, else OMP_NUM_THREADS,
    else min(16, cpu count) (rows are independent: the count never changes a
    result)."""
    for var in ("ATTN_ORACLE_THREADS", "OMP_NUM_THREADS"):
        v = os.environ.get(var, "")
        if v.isdigit() and int(v) > 0:
            return int(v)
    return max(1, min(16, os.cpu_count() or 1))


def attention(q, k, v, scale: float, nthreads: int | None = None):
    """Attention over [..., N, d] tensors (leading dims are heads).

    q: [*, nq, d], k/v: [*, nk, d] with the same leading dims.  Values are taken
    exactly as given (widened to double).  Returns (O [*, nq, d], ml [*, nq, 2]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    nq, d = q.shape[-2:]
    nk = k.shape[-2]
    assert k.shape[:-2] == lead and v.shape == k.shape and k.shape[-1] == d
    bh = int(np.prod(lead)) if lead else 1
    o = np.empty(q.shape, np.float64)
    ml = np.empty(lead + (nq, 2), np.float64)
    if nthreads is None:
        nthreads = default_threads()
    rc = _load().oracle_attention(_dp(q), _dp(k), _dp(v), bh, nq, nk, d, float(scale),
                                  _dp(o), _dp(ml), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed with code {rc}")
    return o, ml
