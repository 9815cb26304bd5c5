"""Helpers shared by the GPU tests: seeded inputs to device tensors, oracle
references, and the acceptance bounds."""
from __future__ import annotations

import numpy as np

import oracle
from attention_attn_stats_amd import synth

# acceptance bounds against the float64 oracle
TOL = {
    "f16": dict(max=5e-3, mean=5e-4),
    "bf16": dict(max=4e-2, mean=4e-3),
    "f32": dict(max=1e-5, mean=1e-6),
}
STATS_RTOL = 1e-3
# m is held to STATS_RTOL relative to |m_ref|, with |m_ref| floored at M_FLOOR:
# a row whose largest logit is within 0.01 of zero is held to 1e-5 absolute
# (a relative error of a quantity near zero says nothing about the kernel)
M_FLOOR = 1e-2


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda().contiguous()


def from_device(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return synth.widen(t.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    return t.detach().cpu().double().numpy()


def reference(q, k, v, dtype: str, scale: float, rows=None):
    """Oracle O and (m, l) on the exact element values (optionally a subset of query rows)."""
    qd, kd, vd = (synth.widen(x, dtype) for x in (q, k, v))
    if rows is not None:
        qd = qd[:, :, rows]
    return oracle.attention(qd, kd, vd, scale)


def assert_close_o(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str, what: str = ""):
    err = np.abs(o_gpu - o_ref)
    tol = TOL[dtype]
    mx, mean = float(err.max()), float(err.mean())
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    assert mx <= tol["max"] and mean <= tol["mean"], (
        f"{what}: max abs err {mx:.3e} (bound {tol['max']:.0e}), mean {mean:.3e} (bound {tol['mean']:.0e})")
    return mx, mean


def assert_close_ml(ml_gpu: np.ndarray, ml_ref: np.ndarray, what: str = ""):
    m, l = ml_gpu[..., 0], ml_gpu[..., 1]
    mr, lr = ml_ref[..., 0], ml_ref[..., 1]
    em = np.abs(m - mr) / np.maximum(M_FLOOR, np.abs(mr))
    el = np.abs(l - lr) / lr
    assert np.isfinite(ml_gpu).all(), f"{what}: non-finite stats"
    assert em.max() <= STATS_RTOL, f"{what}: m rel err {em.max():.3e}"
    assert el.max() <= STATS_RTOL, f"{what}: l rel err {el.max():.3e}"
    return float(em.max()), float(el.max())


def sample_rows(nq: int, n: int, seed: int) -> np.ndarray:
    """First, last and n-2 seeded random query rows, sorted."""
    r = np.random.default_rng(seed)
    rows = set([0, nq - 1]) | set(int(x) for x in r.choice(nq, size=min(n, nq) - 2, replace=False))
    return np.array(sorted(rows))
