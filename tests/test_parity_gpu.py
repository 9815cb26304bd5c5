"""GPU parity: every entry point of libattn.so against the float64 oracle on
the seeded SD UNet attention workloads (full outputs where the oracle is
cheap, sampled query rows at the two large self-attention sizes), in the
element types the library supports, plus ragged and degenerate shapes."""
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
