"""Pins of the group-normalisation and GELU-gated-product oracle
(oracle/unet_ops.c) to things fixed outside it: a 60-digit series for the
error function, textbook values of the normal distribution, SciPy's
independent normal-CDF routine, PyTorch's float64 group_norm, exact rational
arithmetic on tiny groups, closed forms and invariants.  The pages print no
worked example for either kernel, so no pin comes from the pages' numbers.

The readings pinned here (the pages name the operations, not their formulas):
group statistics over the C/G consecutive channels of a group and all spatial
positions, biased variance, eps inside the square root, per-channel affine;
gelu(x) = x Phi(x) with the error function; the gated product takes the first
half of a row as the value and the second half as the gate."""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import unet_ops as ops


# ---- the error function, independently ---------------------------------
def _erf_series(x: Decimal) -> Decimal:
    """erf(x) = 2/sqrt(pi) sum_n (-1)^n x^(2n+1) / (n! (2n+1)), to ~60 digits."""
    getcontext().prec = 80
    pi = Decimal("3.14159265358979323846264338327950288419716939937510582097494459230781640628620899")
    term = x  # x^(2n+1) (-1)^n / n!
    total = Decimal(0)
    n = 0
    while True:
        add = term / (2 * n + 1)
        total += add
        if n > 10 and abs(add) < Decimal("1e-70"):
            break
        n += 1
        term = -term * x * x / n
    return 2 / pi.sqrt() * total


def _gelu_exact(x: float) -> float:
    getcontext().prec = 80
    xd = Decimal(x)
    return float(xd / 2 * (1 + _erf_series(xd / Decimal(2).sqrt())))


@pytest.mark.parametrize("x", [0.0, 0.5, -0.5, 1.0, -1.0, 1.959963984540054, -2.25, 3.0, -3.0, 4.5, -5.5])
def test_gelu_matches_series(x):
    # double rounding of x / sqrt 2 alone moves Phi(x) by about x^2 * 1.1e-16
    # relative in the lower tail, hence the x^2 in the bound
    want = _gelu_exact(x)
    assert abs(ops.gelu1(x) - want) <= (2 + x * x) * 2.5e-16 * abs(want), (x, ops.gelu1(x), want)


def test_gelu_textbook_values():
    # Phi(1) = 0.8413447460685429..., Phi(-1) = 0.1586552539314571...,
    # Phi(1.959963984540054) = 0.975 (the two-sided 95 % point)
    assert ops.gelu1(1.0) == pytest.approx(0.8413447460685429, rel=1e-15)
    assert ops.gelu1(-1.0) == pytest.approx(-0.15865525393145707, rel=1e-14)
    z = 1.959963984540054
    assert ops.gelu1(z) / z == pytest.approx(0.975, rel=1e-15)
    assert ops.gelu1(0.0) == 0.0


def test_gelu_against_scipy_ndtr():
    from scipy.special import ndtr
    x = np.linspace(-12, 12, 4801)
    y = ops.gelu(x)
    want = x * ndtr(x)
    assert np.all(np.abs(y - want) <= (2 + x * x) * 4e-16 * np.abs(want) + 1e-300), \
        np.max(np.abs(y - want) / np.maximum(np.abs(want), 1e-300))


def test_gelu_symmetry_and_tails():
    x = np.linspace(-8, 8, 1601)
    # Phi(x) + Phi(-x) = 1  =>  gelu(x) - gelu(-x) = x
    assert np.allclose(ops.gelu(x) - ops.gelu(-x), x, rtol=0, atol=1e-15)
    assert ops.gelu1(40.0) == 40.0
    assert abs(ops.gelu1(-40.0)) < 1e-300


# ---- the gated product ---------------------------------------------------
def test_geglu_value_first_gate_second():
    # [value | gate] = [2 | 1] -> 2 * gelu(1); the swapped reading would give gelu(2)
    out = ops.geglu(np.array([[2.0, 1.0]]))
    assert out.shape == (1, 1)
    assert out[0, 0] == pytest.approx(2 * _gelu_exact(1.0), rel=1e-15)
    assert abs(out[0, 0] - _gelu_exact(2.0)) > 0.2


def test_geglu_column_pairing():
    # out[:, j] pairs value column j with gate column F + j (not a reversed or shifted gate)
    from scipy.special import ndtr
    v = np.array([[1.0, 10.0, 100.0, 1000.0]])
    g = np.array([[-2.0, -0.5, 0.75, 3.0]])
    out = ops.geglu(np.concatenate([v, g], axis=1))
    want = v * g * ndtr(g)
    assert np.allclose(out, want, rtol=1e-14, atol=0)


def test_geglu_linear_in_value_and_zero_gate():
    rng = np.random.default_rng(5)
    v, g = rng.normal(size=(7, 33)), rng.normal(size=(7, 33)) * 3
    base = ops.geglu(np.concatenate([v, g], axis=1))
    assert np.allclose(ops.geglu(np.concatenate([-2.5 * v, g], axis=1)), -2.5 * base, rtol=1e-14, atol=1e-15)
    assert np.all(ops.geglu(np.concatenate([v, np.zeros_like(g)], axis=1)) == 0.0)
    big = ops.geglu(np.concatenate([v, np.full_like(g, 50.0)], axis=1))
    assert np.allclose(big, 50.0 * v, rtol=1e-15, atol=0)


def test_geglu_rejects_bad_sizes():
    with pytest.raises(AssertionError):
        ops.geglu(np.zeros((2, 3)))


# ---- group normalisation -----------------------------------------------
@pytest.mark.parametrize("shape,groups,eps", [((2, 32, 5, 3), 32, 1e-5), ((2, 64, 4, 4), 32, 1e-6),
                                              ((1, 6, 7, 1), 3, 1e-5), ((3, 8, 2, 5), 1, 0.1),
                                              ((1, 12, 3, 3), 12, 1e-5)])
def test_group_norm_against_torch_float64(shape, groups, eps):
    import torch
    rng = np.random.default_rng(sum(shape) + groups)
    x = rng.normal(size=shape) * 3 + 1.5
    gamma = rng.normal(size=shape[1])
    beta = rng.normal(size=shape[1])
    y, mean, rstd = ops.group_norm(x, groups, gamma, beta, eps)
    want = torch.nn.functional.group_norm(torch.from_numpy(x), groups, torch.from_numpy(gamma),
                                          torch.from_numpy(beta), eps).numpy()
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12), np.max(np.abs(y - want))
    xs = x.reshape(shape[0], groups, -1)
    assert np.allclose(mean, xs.mean(axis=2), rtol=1e-13, atol=1e-14)
    assert np.allclose(rstd, 1 / np.sqrt(xs.var(axis=2) + eps), rtol=1e-12)


def test_group_norm_two_values_closed_form():
    # a group holding a and b equally often: mean (a+b)/2, var ((a-b)/2)^2,
    # y = +-(a-b)/2 / sqrt(var + eps) * gamma + beta
    a, b, eps = 3.0, -1.0, 0.25
    x = np.array([[[a, b], [b, a]], [[7.0, 7.0], [7.0, 7.0]]]).reshape(1, 4, 2)  # C=4, G=2, HW=2
    gamma = np.array([2.0, -1.0, 0.5, 3.0])
    beta = np.array([0.25, 0.5, -1.0, 4.0])
    y, mean, rstd = ops.group_norm(x, 2, gamma, beta, eps)
    half = (a - b) / 2
    r = 1 / math.sqrt(half * half + eps)
    assert mean[0, 0] == 1.0 and rstd[0, 0] == pytest.approx(r, rel=1e-15)
    want0 = np.array([[half * r * 2 + 0.25, -half * r * 2 + 0.25], [-half * r * -1 + 0.5, half * r * -1 + 0.5]])
    assert np.allclose(y[0, :2], want0, rtol=1e-15, atol=1e-15)
    # the constant group: y is beta exactly, rstd = 1/sqrt(eps)
    assert np.all(y[0, 2] == -1.0) and np.all(y[0, 3] == 4.0)
    assert mean[0, 1] == 7.0 and rstd[0, 1] == pytest.approx(2.0, rel=1e-15)


def test_group_norm_exact_rationals():
    # mean and variance by exact rational arithmetic on a small group
    vals = [Fraction(1, 3), Fraction(-5, 7), Fraction(2), Fraction(11, 13), Fraction(-1, 9), Fraction(3, 4)]
    x = np.array([float(v) for v in vals]).reshape(1, 3, 2)  # C=3, one group, HW=2
    xr = [Fraction(float(v)) for v in vals]  # the exact double values
    mean = sum(xr) / len(xr)
    var = sum((v - mean) ** 2 for v in xr) / len(xr)
    eps = Fraction(1, 1000)
    getcontext().prec = 60
    rstd = 1 / (Decimal(var.numerator) / Decimal(var.denominator) + Decimal(eps.numerator) / Decimal(eps.denominator)).sqrt()
    y, m, r = ops.group_norm(x, 1, None, None, float(eps))
    assert m[0, 0] == pytest.approx(float(mean), rel=1e-15)
    assert r[0, 0] == pytest.approx(float(rstd), rel=1e-14)
    for i, v in enumerate(xr):
        want = float((Decimal(v.numerator) / Decimal(v.denominator) - Decimal(mean.numerator) / Decimal(mean.denominator)) * rstd)
        assert y.reshape(-1)[i] == pytest.approx(want, rel=1e-13, abs=1e-15)


def test_group_norm_invariances():
    rng = np.random.default_rng(9)
    x = rng.normal(size=(2, 16, 6, 6))
    y, _, _ = ops.group_norm(x, 4, eps=0.0)
    # a positive scale and a shift of the whole input change nothing when eps = 0
    y2, _, _ = ops.group_norm(3.5 * x - 12.0, 4, eps=0.0)
    assert np.allclose(y, y2, rtol=0, atol=1e-12)
    # normalised groups: mean 0, mean square var / (var + eps)
    eps = 0.3
    y3, _, _ = ops.group_norm(x, 4, eps=eps)
    g = y3.reshape(2, 4, -1)
    var = x.reshape(2, 4, -1).var(axis=2)
    assert np.allclose(g.mean(axis=2), 0, atol=1e-14)
    assert np.allclose((g * g).mean(axis=2), var / (var + eps), rtol=1e-13)


def test_group_norm_groups_are_consecutive_channels():
    # C = 4, G = 2: channels {0, 1} form group 0, {2, 3} group 1.  Changing
    # channel 1 may move group 0's outputs only.
    rng = np.random.default_rng(3)
    x = rng.normal(size=(1, 4, 5))
    x2 = x.copy()
    x2[0, 1] += rng.normal(size=5) * 4
    y, _, _ = ops.group_norm(x, 2)
    y2, _, _ = ops.group_norm(x2, 2)
    assert np.array_equal(y[0, 2:], y2[0, 2:])
    assert not np.allclose(y[0, 0], y2[0, 0])


def test_group_norm_rejects_bad_sizes():
    with pytest.raises(ValueError):
        ops.group_norm(np.zeros((1, 6, 4)), 4)
    with pytest.raises(ValueError):
        ops.group_norm(np.zeros((1, 6, 4)), 3, eps=-1.0)
