"""GPU parity of the strided entry points (attn_*_strided) on the layouts a
UNet attention block hands over without a transpose:

* [B, N, H*d] activations viewed as [B, H, N, d] (head stride d, row stride
  H*d) for q, k, v and out;
* one packed [B, N, 3, H, d] projection output split into q, k, v;
* rows padded past d (a slice of a wider buffer), with the padding of the
  output buffer checked untouched;
* k and v shared by every batch element (batch stride 0).

Every case is compared with the float64 oracle within the element type's
bound, and with the dense entry points on the same values: the kernels only
address memory differently, so the results must be bitwise equal."""
import numpy as np
import pytest

from attention_attn_stats_amd import synth
from attention_attn_stats_amd.configs import CONFIGS, Config
from gpu_util import assert_close_ml, assert_close_o, from_device, reference, sample_rows, to_device

pytestmark = pytest.mark.gpu

FORMS = ("pf", "flash", "auto")


def _run(q, k, v, form, scale, out=None):
    """(O, ml) of one form; ml is None for 'auto' (its statistics are optional)."""
    import attention_attn_stats_amd as attn
    if form == "pf":
        ml = attn.stats(q, k, scale=scale)
        return attn.pv(q, k, v, ml, out=out, scale=scale), ml
    if form == "flash":
        return attn.flash(q, k, v, out=out, want_ml=True, scale=scale)
    return attn.forward(q, k, v, out=out, scale=scale)[0], None


def _bnhd(x: np.ndarray, dtype: str):
    """A [B, H, N, d] array as a view of a [B, N, H*d] device tensor."""
    t = to_device(np.ascontiguousarray(x.transpose(0, 2, 1, 3)), dtype)  # [B, N, H, d]
    return t.transpose(1, 2)


def _check_case(q, k, v, tq, tk, tv, dtype, scale, what, out=None):
    import torch
    dq, dk, dv = (to_device(np.ascontiguousarray(x), dtype) for x in (q, k, v))
    o_ref, ml_ref = reference(q, k, v, dtype, scale)
    for form in FORMS:
        o, ml = _run(tq, tk, tv, form, scale, out=out)
        o_dense, ml_dense = _run(dq, dk, dv, form, scale)
        torch.cuda.synchronize()
        assert o.stride(3) == 1
        assert_close_o(from_device(o), o_ref, dtype, f"{what}/{form}")
        assert torch.equal(o.contiguous(), o_dense), f"{what}/{form}: strided O differs from dense O"
        if ml is not None:
            assert_close_ml(from_device(ml), ml_ref, f"{what}/{form}")
            assert torch.equal(ml, ml_dense), f"{what}/{form}: strided stats differ from dense"
    return o


@pytest.mark.parametrize("name", ["sd512_cross", "level2_self", "level3_self", "level4_self"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bnhd_views(name, dtype):
    cfg = CONFIGS[name]
    q, k, v = cfg.inputs(dtype)
    tq, tk, tv = (_bnhd(x, dtype) for x in (q, k, v))
    assert tq.stride() == (cfg.Nq * cfg.H * cfg.d, cfg.d, cfg.H * cfg.d, 1)
    o = _check_case(q, k, v, tq, tk, tv, dtype, cfg.scale, f"{name}/{dtype} [B,N,H*d]")
    assert o.stride() == tq.stride(), "the default output takes q's layout"


def test_bnhd_views_f32():
    cfg = Config("strided_f32", 81, 2, 3, 100, 70, 80, "f32")
    q, k, v = cfg.inputs()
    _check_case(q, k, v, *(_bnhd(x, "f32") for x in (q, k, v)), "f32", cfg.scale, "f32 [B,N,H*d]")


@pytest.mark.parametrize("d", [40, 80, 160])
def test_packed_qkv(d):
    import torch
    dtype, B, H, N = "f16", 2, 3, 333
    cfg = Config("packed", 82 + d, B, H, N, N, d, dtype)
    q, k, v = cfg.inputs()
    packed = np.stack([x.transpose(0, 2, 1, 3) for x in (q, k, v)], axis=2)  # [B, N, 3, H, d]
    t = to_device(np.ascontiguousarray(packed), dtype)
    tq, tk, tv = (t[:, :, i].transpose(1, 2) for i in range(3))
    assert tk.stride() == (N * 3 * H * d, d, 3 * H * d, 1)
    out = torch.empty((B, N, H, d), device="cuda", dtype=torch.float16).transpose(1, 2)
    _check_case(q, k, v, tq, tk, tv, dtype, cfg.scale, f"packed qkv d{d}", out=out)


@pytest.mark.parametrize("shape", [(1, 2, 130, 77, 40), (2, 1, 65, 200, 80), (1, 1, 1, 1, 160),
                                   (1, 2, 257, 3, 40)], ids=lambda s: "x".join(map(str, s)))
def test_padded_rows_leave_padding_alone(shape):
    import torch
    B, H, Nq, Nk, d = shape
    dtype, pad = "f16", 24
    cfg = Config("padded", 90 + sum(shape), B, H, Nq, Nk, d, dtype)
    q, k, v = cfg.inputs()

    def padded(x):
        buf = np.zeros(x.shape[:3] + (d + pad,), dtype=x.dtype)
        buf[..., :d] = x
        return to_device(buf, dtype)[..., :d]

    tq, tk, tv = (padded(x) for x in (q, k, v))
    assert tq.stride(2) == d + pad
    sentinel = 1234.0
    buf = torch.full((B, H, Nq, d + pad), sentinel, device="cuda", dtype=torch.float16)
    _check_case(q, k, v, tq, tk, tv, dtype, cfg.scale, f"padded rows {shape}", out=buf[..., :d])
    torch.cuda.synchronize()
    assert bool((buf[..., d:] == sentinel).all()), "a write landed in the row padding"


def test_kv_shared_across_batch():
    import torch
    dtype, B, H, Nq, Nk, d = "f16", 3, 2, 200, 77, 40
    q = synth.tensor(101, (B, H, Nq, d), dtype)
    k1 = synth.tensor(102, (1, H, Nk, d), dtype)
    v1 = synth.tensor(103, (1, H, Nk, d), dtype)
    tk = to_device(k1, dtype).expand(B, H, Nk, d)
    tv = to_device(v1, dtype).expand(B, H, Nk, d)
    assert tk.stride(0) == 0
    k, v = np.broadcast_to(k1, (B, H, Nk, d)), np.broadcast_to(v1, (B, H, Nk, d))
    _check_case(q, k, v, _bnhd(q, dtype), tk, tv, dtype, float(np.float32(1 / np.sqrt(d))),
                "k, v shared by the batch")
    torch.cuda.synchronize()


def test_sd512_self_bnhd_sampled_rows():
    """The 64x64-latent self-attention in the [B, N, H*d] layout at full size:
    bitwise equal to the dense run, and sampled rows against the oracle."""
    import torch
    cfg = CONFIGS["sd512_self"]
    q, k, v = cfg.inputs()
    tq, tk, tv = (_bnhd(x, cfg.dtype) for x in (q, k, v))
    dq, dk, dv = (to_device(x, cfg.dtype) for x in (q, k, v))
    rows = sample_rows(cfg.Nq, 16, seed=cfg.index)
    o_ref, ml_ref = reference(q, k, v, cfg.dtype, cfg.scale, rows)
    for form in ("pf", "flash"):
        o, ml = _run(tq, tk, tv, form, cfg.scale)
        o_dense, ml_dense = _run(dq, dk, dv, form, cfg.scale)
        torch.cuda.synchronize()
        assert torch.equal(o.contiguous(), o_dense), f"{form}: strided O differs from dense O"
        assert torch.equal(ml, ml_dense)
        assert_close_o(from_device(o)[:, :, rows], o_ref, cfg.dtype, f"sd512_self [B,N,H*d] {form}")
        assert_close_ml(from_device(ml)[:, :, rows], ml_ref, f"sd512_self [B,N,H*d] {form}")


def test_bad_layouts_are_rejected_before_launch():
    import torch
    import attention_attn_stats_amd as attn
    from attention_attn_stats_amd._lib import AttnError
    d = 40
    q = torch.zeros((1, 1, 16, d + 4), device="cuda", dtype=torch.float16)[..., :d]  # row stride 44
    k = torch.zeros((1, 1, 16, d), device="cuda", dtype=torch.float16)
    with pytest.raises(AttnError, match="invalid argument"):
        attn.flash(q, k, k, scale=0.1)
    with pytest.raises(AttnError, match="invalid argument"):
        attn.stats(q, k, scale=0.1)
    with pytest.raises(ValueError):
        attn.flash(k, k, k, out=torch.zeros((1, 1, 1, d), device="cuda", dtype=torch.float16).expand(1, 1, 16, d))
    with pytest.raises(ValueError):
        attn.scores(torch.zeros((1, 1, 16, d + 8), device="cuda", dtype=torch.float16)[..., :d], k)
