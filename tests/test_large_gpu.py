"""Attention at the size limits of the C ABI, where 32-bit byte offsets would
overflow: one head whose K and V each span more than 2 GiB (2^25 + 77 keys),
Q and O spanning more than 2 GiB (2^25 query rows), 4096 heads, and a single
query over 2^19 keys.  Inputs are seeded device tensors (torch's generator);
results are checked against closed forms computed in float64 and against the
float64 oracle on sampled rows and heads."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import assert_close_ml, assert_close_o, from_device

pytestmark = pytest.mark.gpu

D = 40
SCALE = float(np.float32(1 / math.sqrt(D)))


def _gen(seed):
    import torch
    return torch.Generator(device="cuda").manual_seed(seed)


def test_keys_beyond_two_gib_in_one_head():
    """K = 0 except one key k* near the end: every other score is 0, so
    O_i = (S_v + e^{s*_i} v*) / (Nk - 1 + e^{s*_i}) with S_v the sum of the
    other V rows, m_i = s*_i, l_i = (Nk - 1) e^{-s*_i} + 1.  The queries put
    e^{s*} at about Nk / 77, Nk and 77 Nk, so both terms matter."""
    import torch
    import attention_attn_stats_amd as attn
    Nq, Nk = 64, (1 << 25) + 77
    js = Nk - 5
    g = _gen(11)
    q = torch.randn((1, 1, Nq, D), device="cuda", generator=g).half()
    q[0, 0, :, 0] = torch.tensor([0.75, 1.0, 1.25], device="cuda").repeat(Nq // 3 + 1)[:Nq].half()
    t = math.log(Nk) / (SCALE * 1.0)
    k = torch.zeros((1, 1, Nk, D), device="cuda", dtype=torch.float16)
    k[0, 0, js, 0] = t
    v = torch.randn((1, 1, Nk, D), device="cuda", generator=g).half()
    assert k.numel() * 2 > (1 << 31) and v.numel() * 2 > (1 << 31)
    # closed form in float64 from the exact fp16 values
    qd = q[0, 0].double().cpu().numpy()
    kstar = k[0, 0, js].double().cpu().numpy()
    vstar = v[0, 0, js].double().cpu().numpy()
    sv = (v[0, 0].double().sum(dim=0).cpu().numpy() - vstar)
    s_star = SCALE * (qd @ kstar)
    w = np.exp(s_star)
    o_exp = (sv[None, :] + w[:, None] * vstar[None, :]) / (Nk - 1 + w)[:, None]
    ml_exp = np.stack([s_star, (Nk - 1) * np.exp(-s_star) + 1.0], axis=-1)
    for form in ("flash", "pf"):
        if form == "flash":
            o, ml = attn.flash(q, k, v, want_ml=True, scale=SCALE)
        else:
            ml = attn.stats(q, k, scale=SCALE)
            o = attn.pv(q, k, v, ml, scale=SCALE)
        torch.cuda.synchronize()
        oh = from_device(o)[0, 0]
        err = np.abs(oh - o_exp)
        bound = 2.0 ** -11 * np.abs(o_exp) + 2e-6
        if form == "pf":
            # the second pass forms P against the exact row max, so the 2^25
            # equal small weights e^{-s*} (down to 4e-10) land in fp16's
            # subnormal range and share one rounding of up to 2^-25: their
            # sum moves by up to 2^-25 |S_v| / l.  The single pass adds them
            # up before the large key arrives (P = 1) and rescales in fp32.
            l = (Nk - 1) * np.exp(-s_star) + 1.0
            bound = bound + 2.0 ** -25 * np.abs(sv)[None, :] / l[:, None]
        assert (err <= bound).all(), f"{form}: worst err/bound {np.max(err / bound):.2f}"
        assert_close_ml(from_device(ml)[0, 0], ml_exp, f"{form} stats over 2^25 keys")
        print(form, "max err", err.max(), flush=True)


def test_query_rows_beyond_two_gib():
    import torch
    import attention_attn_stats_amd as attn
    Nq, Nk = 1 << 25, 100
    g = _gen(12)
    q = torch.randn((1, 1, Nq, D), device="cuda", generator=g).half()
    k = torch.randn((1, 1, Nk, D), device="cuda", generator=g).half()
    v = torch.randn((1, 1, Nk, D), device="cuda", generator=g).half()
    assert q.numel() * 2 > (1 << 31)
    rows = np.array([0, 3, 1 << 24, (1 << 24) + 12345, Nq - 257, Nq - 1])
    qs = q[0, 0, torch.as_tensor(rows, device="cuda")].double().cpu().numpy()
    kd, vd = k[0, 0].double().cpu().numpy(), v[0, 0].double().cpu().numpy()
    o_ref, ml_ref = oracle.attention(qs[None], kd[None], vd[None], SCALE)
    for form in ("flash", "pf"):
        if form == "flash":
            o, ml = attn.flash(q, k, v, want_ml=True, scale=SCALE)
        else:
            ml = attn.stats(q, k, scale=SCALE)
            o = attn.pv(q, k, v, ml, scale=SCALE)
        torch.cuda.synchronize()
        sel = torch.as_tensor(rows, device="cuda")
        assert_close_o(from_device(o[0, 0, sel])[None], o_ref, "f16", f"{form} rows past 2 GiB")
        assert_close_ml(from_device(ml[0, 0, sel])[None], ml_ref, f"{form} rows past 2 GiB")
        del o, ml


def test_four_thousand_heads():
    import torch
    import attention_attn_stats_amd as attn
    B, H, N, d = 64, 64, 200, 80
    g = _gen(13)
    q, k, v = (torch.randn((B, H, N, d), device="cuda", generator=g).half() for _ in range(3))
    scale = float(np.float32(1 / math.sqrt(d)))
    o_fl, ml_fl = attn.flash(q, k, v, want_ml=True, scale=scale)
    ml_pf = attn.stats(q, k, scale=scale)
    o_pf = attn.pv(q, k, v, ml_pf, scale=scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (0, 63), (31, 17), (63, 0), (63, 63)):
        qd, kd, vd = (x[b, h].double().cpu().numpy() for x in (q, k, v))
        o_ref, ml_ref = oracle.attention(qd[None], kd[None], vd[None], scale)
        for name, o, ml in (("flash", o_fl, ml_fl), ("pf", o_pf, ml_pf)):
            assert_close_o(from_device(o[b, h])[None], o_ref, "f16", f"{name} head ({b}, {h})")
            assert_close_ml(from_device(ml[b, h])[None], ml_ref, f"{name} head ({b}, {h})")


@pytest.mark.parametrize("d", [40, 80, 160])
def test_single_query_long_context(d):
    # one query per head: the halved workgroup shapes (four key splits at
    # d = 80) walking 2^19 keys
    import torch
    import attention_attn_stats_amd as attn
    B, H, Nk = 2, 2, 1 << 19
    scale = float(np.float32(1 / math.sqrt(d)))
    g = _gen(14 + d)
    q = torch.randn((B, H, 1, d), device="cuda", generator=g).half()
    k = torch.randn((B, H, Nk, d), device="cuda", generator=g).half()
    v = torch.randn((B, H, Nk, d), device="cuda", generator=g).half()
    o_ref, ml_ref = oracle.attention(*(x.double().cpu().numpy() for x in (q, k, v)), scale)
    o, ml = attn.flash(q, k, v, want_ml=True, scale=scale)
    o_only = attn.flash(q, k, v, scale=scale)
    mlp = attn.stats(q, k, scale=scale)
    op = attn.pv(q, k, v, mlp, scale=scale)
    torch.cuda.synchronize()
    for name, oo, mm in (("flash", o, ml), ("flash O only", o_only, None), ("pf", op, mlp)):
        assert_close_o(from_device(oo), o_ref, "f16", f"d={d} {name} one query, 2^19 keys")
        if mm is not None:
            assert_close_ml(from_device(mm), ml_ref, f"d={d} {name} one query, 2^19 keys")
