"""Argument checks of the Python binding: a host tensor, or a tensor of the
wrong shape or type, handed to any entry point raises ValueError in Python,
before a pointer reaches the library (a host pointer given to a kernel would
fault the GPU instead of failing the call)."""
import pytest

pytestmark = pytest.mark.gpu

D = 40


def _qkv(n=16, dtype=None):
    import torch
    dt = dtype or torch.float16
    g = torch.Generator(device="cuda").manual_seed(5)
    return tuple(torch.randn((1, 2, n, D), device="cuda", dtype=dt, generator=g) for _ in range(3))


def test_host_ml_and_out_are_rejected():
    import torch
    import attention_attn_stats_amd as attn
    q, k, v = _qkv()
    ml = attn.stats(q, k)
    host_ml = ml.cpu()
    host_out = torch.empty_like(q, device="cpu")
    with pytest.raises(ValueError):
        attn.pv(q, k, v, host_ml)
    with pytest.raises(ValueError):
        attn.pv(q, k, v, ml, out=host_out)
    with pytest.raises(ValueError):
        attn.flash(q, k, v, out=host_out)
    with pytest.raises(ValueError):
        attn.flash(q, k, v, ml=host_ml)
    with pytest.raises(ValueError):
        attn.stats(q, k, ml=host_ml)
    with pytest.raises(ValueError):
        attn.forward(q, k, v, out=host_out)
    with pytest.raises(ValueError):
        attn.forward(q, k, v, ml=host_ml)
    with pytest.raises(ValueError):
        attn.flash(q, k.cpu(), v)
    torch.cuda.synchronize()


def test_scores_entry_points_reject_host_tensors():
    import torch
    import attention_attn_stats_amd as attn
    q, k, v = _qkv()
    a = attn.scores(q, k)
    ml = attn.scores_stats(a)
    with pytest.raises(ValueError):
        attn.scores_pv(a, ml.cpu(), v)
    with pytest.raises(ValueError):
        attn.scores_pv(a, ml, v, out=torch.empty((1, 2, 16, D), dtype=v.dtype))
    with pytest.raises(ValueError):
        attn.scores_pv(a, ml, v.cpu())
    with pytest.raises(ValueError):
        attn.scores_stats(a, ml=ml.cpu())
    with pytest.raises(ValueError):
        attn.scores(q, k, a=a.cpu())
    # the checked calls still run when every tensor is on the device
    out = attn.scores_pv(a, ml, v)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


def test_wrong_shapes_and_types_are_rejected():
    import torch
    import attention_attn_stats_amd as attn
    q, k, v = _qkv()
    ml = attn.stats(q, k)
    with pytest.raises(ValueError):
        attn.pv(q, k, v, ml[:, :1])
    with pytest.raises(ValueError):
        attn.pv(q, k, v, ml.double())
    with pytest.raises(ValueError):
        attn.flash(q, k, v, out=torch.empty_like(q, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        attn.flash(q, k, v.to(torch.bfloat16))
    torch.cuda.synchronize()
