"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no attention arithmetic: it only turns a seed into tensors of
the documented shapes and distributions, so that the HIP path and the CPU
oracle are fed the very same values.

Recipe (one independent stream per tensor, filled in [B][H][N][d] order):
  * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): state_i = seed + (i + 1) * 0x9E3779B97F4A7C15
    (mod 2^64), output = mix(state_i) with the published 30/27/31 shift,
    0xBF58476D1CE4E5B9 / 0x94D049BB133111EB multiply finaliser;
  * uniform u_i = (output_i >> 11) * 2^-53 in [0, 1);
  * Box-Muller on consecutive pairs: r = sqrt(-2 ln(1 - u_2k)),
    t = 2 pi u_2k+1, n_2k = r cos t, n_2k+1 = r sin t (double precision);
  * multiply by sigma, then round to the target element type: float16 by
    round-to-nearest-even from double; float32 by round-to-nearest-even from
    double; bfloat16 by rounding to float32 first and then
    round-to-nearest-even on the upper 16 bits.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: int) -> np.ndarray:
    """First n outputs of SplitMix64 started at `seed` (uint64 array)."""
    with np.errstate(over="ignore"):
        i = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, n: int) -> np.ndarray:
    """n doubles in [0, 1) with 53 random bits each."""
    return (splitmix64(seed, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, n: int, sigma: float = 1.0) -> np.ndarray:
    """n N(0, sigma^2) doubles by Box-Muller on consecutive uniform pairs."""
    m = (n + 1) // 2
    u = uniform01(seed, 2 * m)
    r = np.sqrt(-2.0 * np.log1p(-u[0::2]))
    t = (2.0 * np.pi) * u[1::2]
    out = np.empty(2 * m, np.float64)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out[:n] * sigma


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round doubles to `dtype` ('f32', 'f16', 'bf16'); returns the rounded
    values as a numpy array of that type (bf16 as uint16 bit patterns)."""
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        f = x.astype(np.float32).view(np.uint32)
        # round-to-nearest-even on the low 16 bits (inputs here are finite)
        bias = ((f >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        return ((f + bias) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of an array produced by round_to."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def tensor(seed: int, shape, dtype: str, sigma: float = 1.0) -> np.ndarray:
    """A seeded N(0, sigma^2) tensor of `shape`, rounded to `dtype`."""
    n = int(np.prod(shape))
    return round_to(normal(seed, n, sigma), dtype).reshape(shape)
