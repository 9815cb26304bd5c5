"""The per-shape choice between the two forms (ATTN_AUTO): the write-up
(attention section) picks FlashAttention or the partially fused softmax per
GPU and head dimension; here both are timed on the device on a shape's first
use and the faster is cached.  These tests check the mechanics: the choice is
one of the two forms, cached per shape, overridden by ATTN_VARIANT, forgotten
by attn_select_reset, and an ATTN_AUTO forward that times a new shape leaves
exactly the chosen form's output (bit for bit)."""
import numpy as np
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


def test_concurrent_callers(monkeypatch):
    """Four host threads, each on its own stream, call ATTN_AUTO on shapes not
    yet timed (two threads share one shape, so they race on its cache entry):
    every result matches the oracle, and the cache ends with one choice per
    shape."""
    import threading
    import torch
    import attention_attn_stats_amd as attn
    from attention_attn_stats_amd import synth
    from gpu_util import assert_close_o, from_device, reference
    monkeypatch.delenv("ATTN_VARIANT", raising=False)
    attn.select_reset()
    shapes = [(1, 2, 300, 257, 40), (1, 2, 200, 129, 80), (1, 1, 96, 65, 160), (1, 2, 300, 257, 40)]
    data = []
    for i, (B, H, Nq, Nk, d) in enumerate(shapes):
        q = synth.tensor(500 + i, (B, H, Nq, d), "f16")
        k = synth.tensor(600 + i, (B, H, Nk, d), "f16")
        v = synth.tensor(700 + i, (B, H, Nk, d), "f16")
        data.append((q, k, v, float(np.float32(1 / np.sqrt(d)))))
    outs, errs = [None] * len(shapes), []

    def work(i):
        try:
            q, k, v, scale = data[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                tq, tk, tv = (to_device(x, "f16") for x in (q, k, v))
                o, _ = attn.forward(tq, tk, tv, variant="auto", scale=scale)
                s.synchronize()
                outs[i] = from_device(o)
        except Exception as e:  # reported below
            errs.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errs, errs
    for i, (q, k, v, scale) in enumerate(data):
        o_ref, _ = reference(q, k, v, "f16", scale)
        assert_close_o(outs[i], o_ref, "f16", f"thread {i} {shapes[i]}")
    for B, H, Nq, Nk, d in shapes:
        assert attn.select(B, H, Nq, Nk, d) in ("pf", "flash")


def test_auto_forward_in_place_over_q(monkeypatch):
    """out = q: an untimed shape must not be timed (repeated runs would read
    their own output); the default variant runs once, and the result equals
    the out-of-place one bit for bit."""
    import torch
    import attention_attn_stats_amd as attn
    from attention_attn_stats_amd import synth
    monkeypatch.delenv("ATTN_VARIANT", raising=False)
    q = synth.tensor(801, (1, 2, 300, 80), "f16")
    k = synth.tensor(802, (1, 2, 333, 80), "f16")
    v = synth.tensor(803, (1, 2, 333, 80), "f16")
    scale = float(np.float32(1 / np.sqrt(80)))
    tq, tk, tv = (to_device(x, "f16") for x in (q, k, v))
    ml = attn.stats(tq, tk, scale=scale)
    ref = attn.pv(tq, tk, tv, ml, scale=scale)  # the default variant at d = 80
    attn.select_reset()
    inplace = tq.clone()
    attn.forward(inplace, tk, tv, variant="auto", out=inplace, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(inplace, ref)
    for form in ("flash", "pf"):  # the explicit forms in place over q as well
        inplace = tq.clone()
        attn.forward(inplace, tk, tv, variant=form, out=inplace, scale=scale)
        torch.cuda.synchronize()
        expect = ref if form == "pf" else attn.flash(tq, tk, tv, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(inplace, expect), form


@pytest.mark.parametrize("name", ["sd512_self", "level2_self"])
def test_select_agrees_with_auto_forward_on_the_workload(name, monkeypatch):
    # attn_select times a shape on seeded stand-in values; an ATTN_AUTO
    # forward times it on the caller's own buffers.  On the seeded workload
    # of a config both must cache the same form.
    import torch
    import attention_attn_stats_amd as attn
    monkeypatch.delenv("ATTN_VARIANT", raising=False)
    monkeypatch.setenv("ATTN_SELECT_ITERS", "9")
    cfg = CONFIGS[name]
    q, k, v = (to_device(x, cfg.dtype) for x in cfg.inputs())
    tdt = q.dtype
    attn.select_reset()
    attn.forward(q, k, v, variant="auto", scale=cfg.scale)
    torch.cuda.synchronize()
    from_forward = attn.select(cfg.B, cfg.H, cfg.Nq, cfg.Nk, cfg.d, tdt)  # the cached choice
    attn.select_reset()
    from_select = attn.select(cfg.B, cfg.H, cfg.Nq, cfg.Nk, cfg.d, tdt)
    print(name, "forward:", from_forward, "select:", from_select, flush=True)
    assert from_forward == from_select
    attn.select_reset()
