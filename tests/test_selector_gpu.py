"""The per-shape choice between the two forms (ATTN_AUTO): the write-up
(attention section) picks FlashAttention or the partially fused softmax per
GPU and head dimension; here both are timed on the device on a shape's first
use and the faster is cached.  These tests check the mechanics: the choice is
one of the two forms, cached per shape, overridden by ATTN_VARIANT, forgotten
by attn_select_reset, and an ATTN_AUTO forward that times a new shape leaves
exactly the chosen form's output (bit for bit)."""
import pytest

from attention_attn_stats_amd.configs import CONFIGS
from gpu_util import to_device

pytestmark = pytest.mark.gpu


def test_choice_is_cached_and_overridden(monkeypatch):
    import attention_attn_stats_amd as attn
    monkeypatch.delenv("ATTN_VARIANT", raising=False)
    attn.select_reset()
    first = attn.select(1, 2, 512, 512, 80)
    assert first in ("pf", "flash")
    assert attn.select(1, 2, 512, 512, 80) == first          # cached
    for forced in ("pf", "flash"):
        monkeypatch.setenv("ATTN_VARIANT", forced)
        assert attn.select(1, 2, 512, 512, 80) == forced      # the override wins over the cache
    monkeypatch.delenv("ATTN_VARIANT")
    assert attn.select(1, 2, 512, 512, 80) == first
    attn.select_reset()
    assert attn.select(1, 2, 512, 512, 80) in ("pf", "flash")  # timed again


@pytest.mark.parametrize("name", ["sd512_cross", "level3_self"])
def test_auto_forward_leaves_the_chosen_forms_output(name, monkeypatch):
    import torch
    import attention_attn_stats_amd as attn
    monkeypatch.delenv("ATTN_VARIANT", raising=False)
    cfg = CONFIGS[name]
    q, k, v = (to_device(x, cfg.dtype) for x in cfg.inputs())
    attn.select_reset()
    o_auto, ml_auto = attn.forward(q, k, v, variant="auto", scale=cfg.scale)  # times both, runs the winner last
    torch.cuda.synchronize()
    chosen = attn.select(cfg.B, cfg.H, cfg.Nq, cfg.Nk, cfg.d, q.dtype)      # the cached choice
    if chosen == "flash":
        ref = attn.flash(q, k, v, scale=cfg.scale)
    else:
        ml = attn.stats(q, k, scale=cfg.scale)
        ref = attn.pv(q, k, v, ml, scale=cfg.scale)
        torch.cuda.synchronize()
        assert torch.equal(ml_auto, ml)
    torch.cuda.synchronize()
    assert torch.equal(o_auto, ref), f"{name}: the auto forward's output is not the {chosen} form's"
    # a second call takes the cached choice without timing, same output
    o2, _ = attn.forward(q, k, v, variant="auto", scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref)
