"""GPU parity: every entry point of libattn.so against the float64 oracle on
the seeded SD UNet attention workloads, every output element compared
(including the two full-size self-attention configs, with sampled-row runs
kept as fast checks), in the element types the library supports, plus ragged
and degenerate shapes."""
import json

import numpy as np
import pytest

from attention_attn_stats_amd.configs import CONFIGS, Config
from gpu_util import (assert_close_ml, assert_close_o, from_device, reference, sample_rows,
                      to_device)

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "tiny8", "sd512_cross", "level2_self", "level3_self", "level4_self"]
LARGE = ["sd512_self", "sd1024_self"]


def _run_all(cfg: Config, dtype: str, rows=None):
    import torch
    import attention_attn_stats_amd as attn
    q, k, v = cfg.inputs(dtype)
    o_ref, ml_ref = reference(q, k, v, dtype, cfg.scale, rows)
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    sel = (lambda t: t[:, :, rows]) if rows is not None else (lambda t: t)
    results = {}
    ml = attn.stats(tq, tk, scale=cfg.scale)
    results["stats"] = assert_close_ml(sel(from_device(ml)), ml_ref, f"{cfg.name}/{dtype}/stats")
    o = attn.pv(tq, tk, tv, ml, scale=cfg.scale)
    results["pv"] = assert_close_o(sel(from_device(o)), o_ref, dtype, f"{cfg.name}/{dtype}/pv")
    o, ml2 = attn.flash(tq, tk, tv, want_ml=True, scale=cfg.scale)
    results["flash"] = assert_close_o(sel(from_device(o)), o_ref, dtype, f"{cfg.name}/{dtype}/flash")
    results["flash_ml"] = assert_close_ml(sel(from_device(ml2)), ml_ref, f"{cfg.name}/{dtype}/flash ml")
    o3 = attn.flash(tq, tk, tv, scale=cfg.scale)
    # the two launches may round the final merge differently, never by more than ~1 ulp
    d = (o3.float() - o.float()).abs().max().item()
    assert d <= 2e-3 * max(1.0, o.float().abs().max().item()), f"flash with / without ml differ by {d}"
    for var in ("pf", "flash", "auto"):
        o, ml3 = attn.forward(tq, tk, tv, variant=var, scale=cfg.scale)
        results[var] = assert_close_o(sel(from_device(o)), o_ref, dtype, f"{cfg.name}/{dtype}/forward {var}")
        if var == "pf":
            assert_close_ml(sel(from_device(ml3)), ml_ref, f"{cfg.name}/{dtype}/forward pf ml")
    torch.cuda.synchronize()
    print(cfg.name, dtype, {k_: tuple(f"{x:.2e}" for x in v_) for k_, v_ in results.items()}, flush=True)
    return results


@pytest.mark.parametrize("name", SMALL)
def test_small_configs_native_dtype(name):
    cfg = CONFIGS[name]
    _run_all(cfg, cfg.dtype)


@pytest.mark.parametrize("name", ["sd512_cross", "level2_self", "level3_self", "level4_self"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_configs_other_dtypes(name, dtype):
    _run_all(CONFIGS[name], dtype)


@pytest.mark.parametrize("name", ["tiny", "tiny8"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiny_in_half_types(name, dtype):
    _run_all(CONFIGS[name], dtype)


@pytest.mark.parametrize("name", LARGE)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_full_size_every_row(name, dtype):
    # the whole output and (m, l) of every form against the oracle (about 1 s
    # of oracle time at 4096 x 4096 and 10-15 s at 16384 x 16384 on 16 threads)
    import time
    cfg = CONFIGS[name]
    t0 = time.perf_counter()
    res = _run_all(cfg, dtype)
    rec = {"config": name, "dtype": dtype, "seconds": round(time.perf_counter() - t0, 1),
           "o_max_mean_abs": {k_: v_ for k_, v_ in res.items() if k_ not in ("stats", "flash_ml")},
           "ml_rel_m_l": {k_: res[k_] for k_ in ("stats", "flash_ml")}}
    print("PARITY " + json.dumps(rec), flush=True)


@pytest.mark.parametrize("name", LARGE)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_full_size_sampled_rows(name, dtype):
    cfg = CONFIGS[name]
    rows = sample_rows(cfg.Nq, 48, seed=cfg.index)
    _run_all(cfg, dtype, rows)


# Ragged and degenerate shapes: query counts that leave partial workgroup
# tiles, key counts that leave a partial key block (or a single key), for each
# head dimension.
RAGGED = [
    # B, H, Nq, Nk, d
    (1, 1, 1, 1, 40),
    (1, 2, 5, 3, 40),
    (2, 3, 77, 77, 40),
    (1, 2, 200, 65, 40),
    (1, 1, 129, 63, 40),
    (2, 1, 300, 129, 80),
    (1, 3, 33, 31, 80),
    (1, 2, 100, 65, 80),   # four key splits of 32 keys: three blocks, the last of one key
    (1, 2, 17, 33, 160),
    (2, 1, 140, 97, 160),
    (1, 1, 64, 1, 160),
]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_ragged_shapes(shape, dtype):
    B, H, Nq, Nk, d = shape
    cfg = Config(f"ragged_{'x'.join(map(str, shape))}", 50 + sum(shape), B, H, Nq, Nk, d, dtype)
    _run_all(cfg, dtype)


# The head-dimension-40 kernel of attn_fa40.hip runs by default only where it
# is the faster one (every workgroup resident, long key ranges); forced here
# onto ragged and degenerate shapes (partial key blocks, one key, partial
# query tiles, more than one round of workgroups).
FA40_FORCED = [(1, 1, 1, 1), (1, 2, 5, 3), (2, 3, 77, 77), (1, 2, 200, 65), (1, 1, 129, 63),
               (1, 2, 300, 2049), (2, 8, 1000, 130), (1, 1, 4096, 64)]


@pytest.mark.parametrize("shape", FA40_FORCED, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fa40_kernel_forced_on_ragged_shapes(shape, dtype, monkeypatch):
    monkeypatch.setenv("ATTN_FA40", "1")
    monkeypatch.setenv("ATTN_SHORT", "0")  # (the short-range kernel would take Nk <= 384)
    B, H, Nq, Nk = shape
    cfg = Config(f"fa40_{'x'.join(map(str, shape))}", 70 + sum(shape), B, H, Nq, Nk, 40, dtype)
    _run_all(cfg, dtype)


# Around the default dispatch boundary of the head-dimension-40 kernel (more
# than 1024 keys, every workgroup resident): the general kernel at 1024 keys,
# the attn_fa40.hip kernel from 1025 on (a one-key last block, a partial one,
# an odd block count that leaves the two key splits uneven).
FA40_BOUNDARY = [(1, 2, 300, 1024), (1, 2, 300, 1025), (2, 1, 257, 1500), (1, 1, 64, 1088)]


@pytest.mark.parametrize("shape", FA40_BOUNDARY, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fa40_dispatch_boundary(shape, dtype, monkeypatch):
    monkeypatch.delenv("ATTN_FA40", raising=False)
    B, H, Nq, Nk = shape
    cfg = Config(f"fa40b_{'x'.join(map(str, shape))}", 90 + sum(shape), B, H, Nq, Nk, 40, dtype)
    _run_all(cfg, dtype)


# The short-key-range kernel of attn_short.hip takes every single pass with
# Nk <= 384 (d = 40) or <= 256 (d = 80, 160).  Its per-wave form (each wave
# loads its own keys) picks key splits per workgroup (1, 2 or 4) and 16-key
# tiles per wave from the shape; its shared form (K and V staged once per
# workgroup of 8 waves) takes at most 96 keys.  These cover one key, partial
# 16-key tiles, an odd tile count (a half-empty PV step), a split left
# without keys, the longest ranges, query tiles past Nq, and grids large
# enough to keep one split; each form is also forced (ATTN_SHORT=w / s).
SHORT = [(1, 1, 1, 1, 40), (1, 2, 5, 3, 40), (2, 3, 77, 77, 40), (1, 2, 200, 97, 40),
         (1, 1, 64, 384, 40), (2, 8, 1000, 77, 40), (1, 2, 17, 256, 80), (2, 1, 100, 129, 80),
         (2, 8, 1000, 50, 80), (1, 1, 1, 1, 160), (1, 3, 33, 31, 160), (2, 2, 100, 65, 160),
         (1, 1, 48, 256, 160), (1, 2, 1000, 16, 160), (2, 8, 300, 200, 160), (1, 2, 300, 96, 160)]


@pytest.mark.parametrize("shape", SHORT, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("form", ["auto", "w", "s"])
def test_short_kernel_on_ragged_shapes(shape, dtype, form, monkeypatch):
    B, H, Nq, Nk, d = shape
    if form == "s" and Nk > 96:
        pytest.skip("the shared form takes at most 96 keys")
    monkeypatch.delenv("ATTN_FA40", raising=False)
    if form == "auto":
        monkeypatch.delenv("ATTN_SHORT", raising=False)
    else:
        monkeypatch.setenv("ATTN_SHORT", form)
    cfg = Config(f"short_{'x'.join(map(str, shape))}", 110 + sum(shape), B, H, Nq, Nk, d, dtype)
    _run_all(cfg, dtype)


# The general single-pass kernel of attn_mfma.hip on short key ranges (which
# the short-range kernel takes by default).
@pytest.mark.parametrize("name", ["sd512_cross", "level3_self", "level4_self"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_general_kernel_forced_on_short_ranges(name, dtype, monkeypatch):
    monkeypatch.setenv("ATTN_SHORT", "0")
    _run_all(CONFIGS[name], dtype)
