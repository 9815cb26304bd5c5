"""GPU parity of the partially fused form over a stored logit matrix
(attn_scores, attn_scores_stats, attn_scores_pv) against the float64 oracle:

* A = scale q k^T element by element, within the float32 accumulation bound
  (a few float32 ulps of scale * sum_c |q_c k_c|);
* the statistics of the GPU's own A against the oracle's statistics of that
  same A (so only the reduction is under test: float32 exp2 and sums), and
  against the oracle's statistics from Q and K within the 1e-3 bound;
* O from the GPU's A and statistics against the oracle's attention, within
  the element type's bound.
Small configs in full, the 512^2 self-attention on sampled query rows, and
ragged shapes (key counts that are not a multiple of 4, single keys)."""
import numpy as np
import pytest

import oracle
from attention_attn_stats_amd import synth
from attention_attn_stats_amd.configs import CONFIGS, Config
from gpu_util import assert_close_ml, assert_close_o, from_device, reference, sample_rows, to_device

pytestmark = pytest.mark.gpu


def _check(cfg: Config, dtype: str, rows=None):
    import torch
    import attention_attn_stats_amd as attn
    q, k, v = cfg.inputs(dtype)
    qd, kd = synth.widen(q, dtype), synth.widen(k, dtype)
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    a = attn.scores(tq, tk, scale=cfg.scale)
    ml = attn.scores_stats(a)
    o = attn.scores_pv(a, ml, tv)
    torch.cuda.synchronize()
    sel = rows if rows is not None else slice(None)
    a_sel = a[:, :, torch.as_tensor(rows, device=a.device)] if rows is not None else a
    a_h = a_sel.cpu().double().numpy()
    ml_h = from_device(ml)[:, :, sel]
    o_h = from_device(o)[:, :, sel]
    scale = float(np.float32(cfg.scale))
    worst_a = worst_ml = 0.0
    for b in range(cfg.B):
        for h in range(cfg.H):
            qh = qd[b, h][sel]
            s_ref = oracle.scores(qh, kd[b, h], scale)
            # float32 accumulation of d exact fp16/bf16 products, then one multiply:
            # at most (d + 2) float32 unit roundoffs of scale * sum_c |q_c k_c|
            bound = (cfg.d + 2) * 2.0 ** -24 * scale * (np.abs(qh) @ np.abs(kd[b, h]).T) + 1e-30
            err = np.abs(a_h[b, h] - s_ref)
            assert (err <= bound).all(), f"{cfg.name}/{dtype} A: worst err/bound {np.max(err / bound):.2f}"
            worst_a = max(worst_a, float(np.max(err / bound)))
            # the reduction alone: statistics of the GPU's own A
            _, m_ref, l_ref = oracle.softmax_rows(a_h[b, h])
            em = np.abs(ml_h[b, h, :, 0] - m_ref) / np.maximum(1.0, np.abs(m_ref))
            el = np.abs(ml_h[b, h, :, 1] - l_ref) / l_ref
            assert em.max() <= 1e-6 and el.max() <= 2e-5, (
                f"{cfg.name}/{dtype} stats of A: m {em.max():.2e}, l {el.max():.2e}")
            worst_ml = max(worst_ml, float(el.max()))
    o_ref, ml_ref = reference(q, k, v, dtype, cfg.scale, rows)
    assert_close_ml(ml_h, ml_ref, f"{cfg.name}/{dtype} scores_stats vs oracle")
    assert_close_o(o_h, o_ref, dtype, f"{cfg.name}/{dtype} scores_pv")
    print(cfg.name, dtype, f"A err/bound {worst_a:.2f}, l rel (same A) {worst_ml:.1e}", flush=True)


@pytest.mark.parametrize("name", ["sd512_cross", "level2_self", "level3_self", "level4_self"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_small_configs(name, dtype):
    _check(CONFIGS[name], dtype)


def test_sd512_self_sampled_rows():
    cfg = CONFIGS["sd512_self"]
    _check(cfg, cfg.dtype, sample_rows(cfg.Nq, 24, seed=cfg.index))


RAGGED = [(1, 1, 1, 1, 40), (1, 2, 5, 3, 40), (2, 1, 130, 77, 40), (1, 1, 64, 129, 80),
          (1, 2, 33, 31, 160), (1, 1, 200, 65, 40)]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_shapes(shape):
    B, H, Nq, Nk, d = shape
    _check(Config(f"ragged_{'x'.join(map(str, shape))}", 70 + sum(shape), B, H, Nq, Nk, d, "f16"), "f16")


def test_stats_pass_is_the_block_split_of_its_input():
    """attn_scores_stats on a hand-built A: rows whose (m, l) are known in closed
    form (logs of small integers, an all-equal row, a single huge entry)."""
    import torch
    import attention_attn_stats_amd as attn
    Nk = 300
    rows = []
    r0 = np.zeros(Nk); rows.append(r0)                                  # m = 0, l = Nk
    r1 = np.full(Nk, -1e4); r1[123] = 5.0; rows.append(r1)              # m = 5, l = 1
    r2 = np.log(np.arange(1, Nk + 1, dtype=np.float64)); rows.append(r2)  # m = log Nk, l = sum j / Nk
    r3 = -np.arange(Nk, dtype=np.float64); rows.append(r3)              # m = 0, l = 1 / (1 - e^-1) (tail e^-300)
    a = torch.tensor(np.stack(rows)[None, None], dtype=torch.float32, device="cuda").contiguous()
    ml = attn.scores_stats(a).cpu().double().numpy()[0, 0]
    a32 = np.stack(rows).astype(np.float32).astype(np.float64)
    want_m = [0.0, 5.0, a32[2].max(), 0.0]
    want_l = [Nk, 1.0, np.exp(a32[2] - a32[2].max()).sum(), 1.0 / (1.0 - np.exp(-1.0))]
    for i in range(4):
        assert abs(ml[i, 0] - want_m[i]) <= 1e-6 * max(1.0, abs(want_m[i])), (i, ml[i], want_m[i])
        assert abs(ml[i, 1] - want_l[i]) <= 2e-5 * want_l[i], (i, ml[i], want_l[i])
