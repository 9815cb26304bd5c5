"""GPU parity of the UNet's group normalisation (attn_group_norm) and
GELU-gated product (attn_geglu) against the float64 oracle (oracle/unet_ops.c),
element by element, within bounds derived from the arithmetic:

* group_norm: output rounding u|y| (u = 2^-11 fp16, 2^-8 bf16, 0 for fp32)
  plus float32 error of the statistics and of the affine step,
  32 * 2^-24 * (|gamma| rstd (|x| + |mean| + sigma) + |beta|);
* geglu: output rounding u|out| (plus 2^-25 for fp16 results below the
  normal range, and (1 + |v g|) 2^-126 for float32 intermediates flushed to
  zero) plus the error of the erfc fit (fractional 1.2e-7) and of its
  float32 evaluation (ten Horner steps over terms up to ~3 in size: below
  1.8e-6 in the base-2 exponent, 1.3e-6 relative), |v| |gelu(g)| (2e-6 +
  1e-7 g^2).

Shapes: the SD 1.x UNet's normalisation and feed-forward sizes at 512x512
(batch 2), both launch forms of the group normalisation (one launch with the
group in one workgroup's registers, at every register depth; two launches over
slices for larger groups, also forced on small ones), ragged and unaligned
sizes (element-wise paths), in-place use, and activations with a large common
offset (mean 100, sigma 1), where a sum-of-squares variance would fail."""
import numpy as np
import pytest

from attention_attn_stats_amd import synth
from oracle import unet_ops as ops

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8, "f32": 0.0}
TORCH_DT = {"f16": "float16", "bf16": "bfloat16", "f32": "float32"}


def _dev(a: np.ndarray, dtype: str):
    """Exact element-type values of a float64 array -> device tensor (and the values)."""
    import torch
    r = synth.round_to(a, dtype)
    w = synth.widen(r, dtype)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(r).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(r))
    return t.cuda(), w


def _host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return synth.widen(t.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    return t.detach().cpu().double().numpy()


# ---- group normalisation -----------------------------------------------
def _gn_case(N, C, HW, G, dtype, seed, mean=0.0, sigma=1.0, affine=True, inplace=False,
             offset_elems=0, eps=1e-5):
    import torch
    import attention_attn_stats_amd as attn
    n = N * C * HW
    # per-channel offsets on top of the common one, as in real activations
    chan = synth.normal(seed + 1, C).reshape(1, C, 1) * 0.5
    x = (synth.normal(seed, n).reshape(N, C, HW) * sigma + mean + chan)
    if offset_elems:
        # an unaligned view: the tensor starts offset_elems elements into its buffer
        buf, xw = _dev(np.concatenate([np.zeros(offset_elems), x.reshape(-1)]), dtype)
        tx = buf[offset_elems:].view(N, C, HW)
        xw = xw[offset_elems:].reshape(N, C, HW)
    else:
        tx, xw = _dev(x, dtype)
    if affine:
        tg, gw = _dev(1.0 + 0.3 * synth.normal(seed + 2, C), dtype)
        tb, bw = _dev(0.2 * synth.normal(seed + 3, C), dtype)
    else:
        tg = tb = gw = bw = None
    y_ref, m_ref, r_ref = ops.group_norm(xw, G, gw, bw, eps)
    out = tx if inplace else None
    y = attn.group_norm(tx, G, tg, tb, eps=eps, out=out)
    torch.cuda.synchronize()
    yh = _host(y)
    ga = np.abs(gw)[None, :, None] if affine else 1.0
    be = np.abs(bw)[None, :, None] if affine else 0.0
    mean_e = np.repeat(m_ref, C // G, axis=1)[:, :, None]
    rstd_e = np.repeat(r_ref, C // G, axis=1)[:, :, None]
    sig_e = 1.0 / rstd_e
    bound = (U[dtype] * np.abs(y_ref) + (2.0 ** -25 if dtype == "f16" else 0.0)
             + 32 * 2.0 ** -24 * (ga * rstd_e * (np.abs(xw) + np.abs(mean_e) + sig_e) + be))
    err = np.abs(yh - y_ref)
    i = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.isfinite(yh).all()
    assert (err <= bound).all(), (f"group_norm N{N} C{C} HW{HW} G{G} {dtype}: element {i} err {err[i]:.3e} "
                                  f"> bound {bound[i]:.3e} (y_ref {y_ref[i]:.4f})")
    return float((err / bound).max())


SD_GN = [  # (C, HW) of the SD 1.x UNet's group normalisations at 512x512, batch 2
    (320, 64 * 64), (640, 64 * 64), (960, 64 * 64), (640, 32 * 32), (1280, 32 * 32),
    (1920, 16 * 16), (1280, 16 * 16), (2560, 8 * 8), (1280, 8 * 8)]


@pytest.mark.parametrize("C,HW", SD_GN, ids=lambda v: str(v))
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_group_norm_sd_shapes(C, HW, dtype):
    r = _gn_case(2, C, HW, 32, dtype, seed=C + HW)
    print(f"gn C{C} HW{HW} {dtype} err/bound {r:.3f}", flush=True)


def test_group_norm_large_groups():
    # 1024x1024 image, decoder input: 640 channels at 128x128: groups of
    # 327680 elements, beyond one workgroup's registers, split over
    # workgroups (one launch while they are all resident, else two)
    import attention_attn_stats_amd as attn
    from attention_attn_stats_amd import _lib
    assert _lib.load().attn_group_norm_workspace_size(1 << 20, 1 << 20, 2, 640, 128 * 128, 32, _lib.F16) > 0
    _gn_case(2, 640, 128 * 128, 32, "f16", seed=7)
    _gn_case(1, 64, 40000, 2, "f32", seed=8)          # f32: 65536-element register limit
    _gn_case(1, 32, 20001, 1, "bf16", seed=9)         # element-wise path beyond 16384 elements
    del attn


@pytest.mark.parametrize("C,HW", [(320, 4096), (64, 100), (1280, 64)], ids=lambda v: str(v))
def test_group_norm_two_launch_path_forced(C, HW, monkeypatch):
    # the two-launch form on groups that would fit one workgroup, through the
    # same entry point (the plan reads ATTN_GN_PATH at every call)
    monkeypatch.setenv("ATTN_GN_PATH", "split")
    for dtype in ("f16", "f32"):
        _gn_case(2, C, HW, 32, dtype, seed=C + HW + 1)


@pytest.mark.parametrize("C,HW", [(320, 4096), (960, 4096), (1280, 1024), (640, 16384), (64, 999)],
                         ids=lambda v: str(v))
def test_group_norm_one_launch_split_forced(C, HW, monkeypatch):
    # groups split over workgroups that exchange moments in one launch
    monkeypatch.setenv("ATTN_GN_PATH", "coop")
    for dtype in ("f16", "bf16", "f32"):
        _gn_case(2, C, HW, 32, dtype, seed=C + HW + 2)


def test_group_norm_bounded_wait_fallback_is_identical(monkeypatch):
    """With no polls allowed, every workgroup that is not last to arrive
    computes all of its group's slice moments itself: the output must be the
    same bits as when the workgroups exchange them."""
    import torch
    import attention_attn_stats_amd as attn
    for shape, dt in (((2, 320, 64 * 64), torch.float16), ((2, 960, 64 * 64), torch.bfloat16),
                      ((2, 64, 999), torch.float32)):
        x = torch.randn(shape, device="cuda", generator=torch.Generator(device="cuda").manual_seed(3)).to(dt)
        monkeypatch.setenv("ATTN_GN_PATH", "coop")
        y0 = attn.group_norm(x, 32)
        monkeypatch.setenv("ATTN_GN_SPIN", "0")
        y1 = attn.group_norm(x, 32)
        monkeypatch.delenv("ATTN_GN_SPIN")
        y2 = attn.group_norm(x, 32)  # and the counters were left ready
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), f"{shape}: the fallback differs"
        assert torch.equal(y0, y2), f"{shape}: a second exchange differs"


@pytest.mark.parametrize("rv_elems", [1000, 9000, 20000, 40000, 70000, 130000])
def test_group_norm_every_register_depth(rv_elems, monkeypatch):
    # groups of about rv_elems fp16 elements in one launch: 1, 2, 4, 8, 16
    # vectors per thread (forced: so few groups would otherwise take two)
    monkeypatch.setenv("ATTN_GN_PATH", "fused")
    _gn_case(2, 2, rv_elems // 8 * 8, 2, "f16", seed=rv_elems)
    _gn_case(1, 4, rv_elems // 16 * 4, 2, "f32", seed=rv_elems + 1)


def test_group_norm_many_groups_one_launch():
    # batch 8: 256 groups fill the chip in one launch
    from attention_attn_stats_amd import _lib
    assert _lib.load().attn_group_norm_workspace_size(1 << 20, 1 << 20, 8, 320, 64 * 64, 32, _lib.F16) == 0
    _gn_case(8, 320, 64 * 64, 32, "f16", seed=31)


def test_group_norm_large_common_offset():
    # mean 100, sigma 1: E[x^2] - E[x]^2 in float32 would lose every digit
    for dtype in ("f32", "bf16"):
        _gn_case(2, 320, 64 * 64, 32, dtype, seed=11, mean=100.0, sigma=1.0)
    _gn_case(1, 64, 1000, 8, "f32", seed=12, mean=-3000.0, sigma=0.5)


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 4, 1, 2), (2, 6, 7, 3), (1, 32, 15, 32), (3, 64, 33, 4),
                                   (1, 5, 4096, 5), (2, 96, 9, 32), (1, 12, 64, 1)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_group_norm_ragged(shape, dtype):
    N, C, HW, G = shape
    _gn_case(N, C, HW, G, dtype, seed=sum(shape), eps=1e-6)


def test_group_norm_forms_agree_and_options():
    # no affine, in place, an unaligned tensor (element-wise path), eps = 0
    _gn_case(2, 320, 32 * 32, 32, "f16", seed=21, affine=False)
    _gn_case(2, 320, 32 * 32, 32, "f16", seed=22, inplace=True)
    _gn_case(2, 320, 64 * 64, 32, "bf16", seed=23, inplace=True)
    _gn_case(2, 64, 256, 32, "f16", seed=24, offset_elems=3)
    _gn_case(1, 32, 4096, 32, "f32", seed=25, offset_elems=1)
    _gn_case(2, 320, 64 * 64, 32, "f32", seed=26, eps=0.0)


def test_group_norm_is_deterministic_and_forms_agree(monkeypatch):
    import torch
    import attention_attn_stats_amd as attn
    x = torch.randn(2, 320, 64, 64, device="cuda", dtype=torch.float16)
    y0 = attn.group_norm(x, 32)
    for _ in range(3):
        assert torch.equal(attn.group_norm(x, 32), y0)
    # the two-launch form merges the moments in another order: the two agree
    # to one rounding of the fp16 output
    monkeypatch.setenv("ATTN_GN_PATH", "split")
    y1 = attn.group_norm(x, 32)
    assert torch.equal(attn.group_norm(x, 32), y1)
    d = (y1.float() - y0.float()).abs()
    assert bool((d <= 2.0 ** -10 * y0.float().abs() + 2.0 ** -24).all()), d.max().item()


def test_group_norm_bad_arguments():
    import torch
    import attention_attn_stats_amd as attn
    from attention_attn_stats_amd._lib import AttnError
    x = torch.zeros(2, 30, 8, device="cuda", dtype=torch.float16)
    with pytest.raises(AttnError, match="invalid argument"):
        attn.group_norm(x, 4)  # 30 channels, 4 groups
    with pytest.raises(AttnError, match="invalid argument"):
        attn.group_norm(x, 3, eps=-1.0)


# ---- GELU-gated product --------------------------------------------------
def _geglu_case(rows, F, dtype, seed, gate_sigma=1.0, offset_elems=0, ramp=False):
    import torch
    import attention_attn_stats_amd as attn
    v = synth.normal(seed, rows * F).reshape(rows, F)
    if ramp:
        g = np.broadcast_to(np.linspace(-14.0, 14.0, F), (rows, F)).copy()
    else:
        g = synth.normal(seed + 1, rows * F).reshape(rows, F) * gate_sigma
    h = np.concatenate([v, g], axis=1)
    if offset_elems:
        buf, hw = _dev(np.concatenate([np.zeros(offset_elems), h.reshape(-1)]), dtype)
        th = buf[offset_elems:].view(rows, 2 * F)
        hw = hw[offset_elems:].reshape(rows, 2 * F)
    else:
        th, hw = _dev(h, dtype)
    ref = ops.geglu(hw)
    out = attn.geglu(th)
    torch.cuda.synchronize()
    oh = _host(out)
    vw, gw = hw[:, :F], hw[:, F:]
    gel = ops.gelu(gw)
    # absolute floors: fp16 results below the normal range are rounded to a
    # 2^-24 spacing; float32 intermediates below 2^-126 may be flushed to zero
    bound = (U[dtype] * np.abs(ref) + (2.0 ** -25 if dtype == "f16" else 0.0)
             + (1.0 + np.abs(vw * gw)) * 2.0 ** -126
             + np.abs(vw) * np.abs(gel) * (2e-6 + 1e-7 * gw * gw))
    err = np.abs(oh - ref)
    i = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.isfinite(oh).all()
    assert (err <= bound).all(), (f"geglu {rows}x{F} {dtype}: element {i} err {err[i]:.3e} > bound {bound[i]:.3e} "
                                  f"(v {vw[i]:.4f}, g {gw[i]:.4f})")
    return float((err / bound).max())


SD_FF = [(8192, 1280), (2048, 2560), (512, 5120), (128, 5120)]  # (tokens, inner dim) at 512x512, batch 2


@pytest.mark.parametrize("rows,F", SD_FF, ids=lambda v: str(v))
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_geglu_sd_shapes(rows, F, dtype):
    r = _geglu_case(rows, F, dtype, seed=rows + F)
    print(f"geglu {rows}x{F} {dtype} err/bound {r:.3f}", flush=True)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_geglu_gate_tails(dtype):
    # gates from -14 to 14 (deep lower tail, where Phi underflows, and the
    # upper tail, where gelu(g) = g)
    _geglu_case(7, 4096, dtype, seed=3, ramp=True)
    _geglu_case(64, 1280, dtype, seed=4, gate_sigma=4.0)


@pytest.mark.parametrize("shape", [(1, 1), (1, 7), (3, 13), (5, 8), (2, 1000), (17, 2561), (1, 16)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_geglu_ragged(shape, dtype):
    _geglu_case(*shape, dtype, seed=sum(shape))


def test_geglu_unaligned_and_odd_sizes():
    import torch
    import attention_attn_stats_amd as attn
    _geglu_case(9, 640, "f16", seed=5, offset_elems=1)
    _geglu_case(9, 640, "bf16", seed=6, offset_elems=5)
    with pytest.raises(ValueError):
        attn.geglu(torch.zeros(4, 7, device="cuda", dtype=torch.float16))  # odd last dim


def test_group_norm_workspace_cache_is_bounded():
    # a workspace per stream, the least recently used dropped beyond the bound;
    # every call still matches the oracle
    import torch
    import attention_attn_stats_amd as attn
    from attention_attn_stats_amd import api
    x = torch.randn((2, 320, 64 * 64), device="cuda", generator=torch.Generator(device="cuda").manual_seed(4)).half()
    ref = attn.group_norm(x, 32)
    for _ in range(api._GN_WS_MAX + 5):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            y = attn.group_norm(x, 32)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
    assert len(api._GN_WS) <= api._GN_WS_MAX


def _random_gn_cases(n=30, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 8, 32]))
        C = G * int(rng.integers(1, 41))
        HW = int(rng.integers(1, 9000)) if i % 3 else int(rng.choice([64, 256, 1024, 4096]))
        N = int(rng.integers(1, 4))
        dtype = ("f16", "bf16", "f32")[i % 3]
        out.append((N, C, HW, G, dtype))
    return out


@pytest.mark.parametrize("case", _random_gn_cases(), ids=lambda c: "x".join(map(str, c[:4])) + f"-{c[4]}")
def test_group_norm_random_shapes(case):
    # seeded random shapes: groups from a handful of elements to ~360000,
    # aligned and ragged spatial sizes, every element type; the plan picks
    # whichever form fits, each checked against the oracle's bound
    N, C, HW, G, dtype = case
    _gn_case(N, C, HW, G, dtype, seed=N * 7919 + C * 104729 + HW * 13 + G)


def _random_geglu_cases(n=20, seed=20261205):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 3000)), int(rng.integers(1, 3000)), ("f16", "bf16", "f32")[i % 3])
            for i in range(n)]


@pytest.mark.parametrize("case", _random_geglu_cases(), ids=lambda c: f"{c[0]}x{c[1]}-{c[2]}")
def test_geglu_random_shapes(case):
    rows, F, dtype = case
    _geglu_case(rows, F, dtype, seed=rows * 31 + F)


@pytest.mark.parametrize("C,HW", [(320, 4096), (960, 4096)], ids=lambda v: str(v))
def test_group_norm_in_place_with_no_wait(C, HW, monkeypatch):
    # in place, with the one-launch split form asked for and no polls
    # allowed: an in-place call must not take a form whose fallback rereads
    # its partners' slices of x (which they may already have overwritten)
    monkeypatch.setenv("ATTN_GN_PATH", "coop")
    monkeypatch.setenv("ATTN_GN_SPIN", "0")
    for dtype in ("f16", "bf16"):
        _gn_case(2, C, HW, 32, dtype, seed=C + HW + 7, inplace=True)
