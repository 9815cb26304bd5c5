"""Element-wise rounding bounds for the 16-bit paths (the fp16 / bf16
tolerance campaign): beyond the fixed acceptance bounds, every output element
of every form must lie within an a-priori bound derived from the arithmetic
the kernels perform, so that an error that stays under the fixed bound only
because the data are benign (a dropped term, a wrong rescale, a rounding step
at the wrong place) still fails.

With u the unit roundoff of the element type (2^-11 fp16, 2^-8 bf16), p the
exact softmax row and O = p V (float64 oracle), an element of the output
carries at most:

* u (p.|v|)    rounding of P to the element type before the P V product;
* u |O|        rounding of the normaliser (the statistics pass and the
               product pass round their P separately), and
* u |O|        rounding of O itself;
* 2 E (p.|v| + |O|)  float32 score error: E = (d + 4) 2^-24 scale max_j
               sum_c |q_c k_jc| + 2^-23 (max|s| + |m|) per row, from the
               accumulation of d products and the fused shift by the max;
* (Nk/16 + 8) 2^-24 (p.|v| + |O|)  float32 accumulation of the product and of l
               over Nk keys in 16-key steps;
* fp16 only: 2^-25 sum over the weights below fp16's normal range
               (exp(s - m) < 2^-14) of (|v_j| + |O|) / l: those are rounded
               to a fixed spacing, not relative to their size;
* the fp16 O-only single pass at head dim 40 (Nk > 1024) only: its scores
  come from Q scaled into exp2 units and rounded to fp16, so E gains
  u scale max_j sum_c |q_c k_jc| + 2^-25 ln 2 max_j sum_c |k_jc| (scaled
  query elements in fp16's subnormal range) + (d + 5) 2^-24 (|m| + 3) (the
  reference, an extra product term);

to first order, plus 1e-7 absolute.  The tests report max(err / bound).
"""
import os

import numpy as np
import pytest

import oracle
from attention_attn_stats_amd import synth
from attention_attn_stats_amd.configs import CONFIGS, Config
from gpu_util import from_device, sample_rows, to_device

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def bound_and_reference(q, k, v, dtype, scale, rows=None):
    """(O_ref, bound) of the same shape [B, H, rows, d]."""
    qd, kd, vd = (synth.widen(x, dtype) for x in (q, k, v))
    if rows is not None:
        qd = qd[:, :, rows]
    B, H, Nq, d = qd.shape
    Nk = kd.shape[2]
    u = U[dtype]
    o_ref = np.empty((B, H, Nq, d))
    bnd = np.empty_like(o_ref)
    bnd_fold = np.empty_like(o_ref)
    for b in range(B):
        for h in range(H):
            s = oracle.scores(qd[b, h], kd[b, h], scale)
            p, m, l = oracle.softmax_rows(s)
            o = oracle.pv(p, vd[b, h])
            pva = oracle.pv(p, np.abs(vd[b, h]))
            qk_abs = (np.abs(qd[b, h]) @ np.abs(kd[b, h]).T).max(axis=1)
            e_s = ((d + 4) * 2.0 ** -24 * scale * qk_abs
                   + 2.0 ** -23 * (np.abs(s).max(axis=1) + np.abs(m)))[:, None]
            e_fold = (u * scale * qk_abs + 2.0 ** -25 * np.log(2.0) * np.abs(kd[b, h]).sum(axis=1).max()
                      + (d + 5) * 2.0 ** -24 * (np.abs(m) + 3.0))[:, None]
            acc = (Nk / 16 + 8) * 2.0 ** -24
            sub = 0.0
            if dtype == "f16":
                tiny = (p * l[:, None] < 2.0 ** -14).astype(np.float64)
                sub = 2.0 ** -25 * (tiny @ np.abs(vd[b, h]) + tiny.sum(axis=1, keepdims=True) * np.abs(o)) / l[:, None]
            o_ref[b, h] = o
            bnd[b, h] = (u * (pva + 2 * np.abs(o)) + (2 * e_s + acc) * (pva + np.abs(o)) + sub + 1e-7)
            bnd_fold[b, h] = bnd[b, h] + 2 * e_fold * (pva + np.abs(o))
    return o_ref, bnd, bnd_fold


def _forms(tq, tk, tv, scale):
    import attention_attn_stats_amd as attn
    ml = attn.stats(tq, tk, scale=scale)
    yield "pf", attn.pv(tq, tk, tv, ml, scale=scale)
    yield "flash", attn.flash(tq, tk, tv, scale=scale)
    yield "flash+ml", attn.flash(tq, tk, tv, want_ml=True, scale=scale)[0]


def _check(q, k, v, dtype, scale, what, rows=None):
    import torch
    o_ref, bnd, bnd_fold = bound_and_reference(q, k, v, dtype, scale, rows)
    # the forms whose kernel folds the scale into the fp16 score product
    fa40 = os.environ.get("ATTN_FA40")
    on_fa40 = q.shape[-1] == 40 and (fa40 == "1" or (fa40 != "0" and k.shape[2] > 1024))
    folded = {"flash"} if (dtype == "f16" and on_fa40) else set()
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    worst = {}
    for form, o in _forms(tq, tk, tv, scale):
        torch.cuda.synchronize()
        og = from_device(o)
        if rows is not None:
            og = og[:, :, rows]
        b_form = bnd_fold if form in folded else bnd
        r = np.abs(og - o_ref) / b_form
        worst[form] = float(r.max())
        i = np.unravel_index(np.argmax(r), r.shape)
        assert r.max() <= 1.0, (f"{what}/{dtype}/{form}: element {i} err {abs(og[i] - o_ref[i]):.3e} "
                                f"exceeds its rounding bound {b_form[i]:.3e}")
    print(what, dtype, {f: f"{x:.3f}" for f, x in worst.items()}, flush=True)


@pytest.mark.parametrize("name", ["sd512_cross", "level2_self", "level3_self", "level4_self", "tiny"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_configs_within_rounding_bound(name, dtype):
    cfg = CONFIGS[name]
    _check(*cfg.inputs(dtype), dtype, cfg.scale, name)


@pytest.mark.parametrize("name", ["sd512_self", "sd1024_self"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_full_size_rows_within_rounding_bound(name, dtype):
    cfg = CONFIGS[name]
    _check(*cfg.inputs(dtype), dtype, cfg.scale, name, sample_rows(cfg.Nq, 12, seed=cfg.index + 5))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("sigma", [0.25, 3.0])
@pytest.mark.parametrize("d", [40, 80, 160])
def test_logit_spread_within_rounding_bound(dtype, sigma, d):
    # flat (sigma 0.25: every weight near 1/Nk) and peaked (sigma 3: scores
    # spread over hundreds) softmax rows, ragged sizes
    cfg = Config("spread", 200 + d + int(sigma * 4), 1, 2, 190, 333, d, dtype, sigma_qk=sigma)
    _check(*cfg.inputs(), dtype, cfg.scale, f"sigma {sigma} d {d}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_large_values_of_v_within_rounding_bound(dtype):
    # |v| up to ~100: the bound scales with p.|v|, the fixed bound would not
    cfg = Config("bigv", 230, 1, 2, 150, 260, 40, dtype, sigma_v=30.0)
    _check(*cfg.inputs(), dtype, cfg.scale, "sigma_v 30")
