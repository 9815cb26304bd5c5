"""GPU properties of the attention path that hold at any size, checked through
the C ABI on inputs built to exercise one behaviour each:

* the softmax weights of a row sum to one: a V whose every row is the same
  vector gives that vector back, and Q = 0 gives the column means of V with
  m = 0 and l = Nk;
* adding one vector u to every key adds scale * q.u to a whole score row,
  which moves m by that amount and leaves O and l unchanged;
* one key far above the rest takes (almost) all the weight, wherever it sits
  in the key sequence (late keys force a rescale of the running state);
* scores that grow along the key sequence make the running max move on every
  block; the result still matches the oracle;
* results are bitwise repeatable, and the same on a side stream as on the
  default stream.
"""
import numpy as np
import pytest

from attention_attn_stats_amd import synth
from attention_attn_stats_amd.configs import CONFIGS
from gpu_util import assert_close_ml, assert_close_o, from_device, reference, to_device

pytestmark = pytest.mark.gpu

FORMS = ("pf", "flash")
# flash_o: the single pass without (m, l) out (the fp16 head-dim-40 kernel
# then takes its folded fast path: scale and reference inside the product)
FORMS_O = FORMS + ("flash_o",)


def _forward(q, k, v, form, scale):
    import attention_attn_stats_amd as attn
    if form == "pf":
        ml = attn.stats(q, k, scale=scale)
        return attn.pv(q, k, v, ml, scale=scale), ml
    if form == "flash_o":
        return attn.flash(q, k, v, scale=scale), None
    return attn.flash(q, k, v, want_ml=True, scale=scale)


def _exact(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the element type and back to float64 (the values the GPU sees)."""
    return synth.widen(synth.round_to(a, dtype), dtype)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("dtype,d", [("f16", 40), ("bf16", 80), ("f16", 160)])
def test_constant_v_rows_come_back(form, dtype, d):
    B, H, Nq, Nk = 1, 2, 150, 333
    q = synth.round_to(synth.normal(11, B * H * Nq * d).reshape(B, H, Nq, d), dtype)
    k = synth.round_to(synth.normal(12, B * H * Nk * d).reshape(B, H, Nk, d), dtype)
    row = synth.normal(13, d) * 2.0
    v = synth.round_to(np.broadcast_to(row, (B, H, Nk, d)).copy(), dtype)
    scale = 1.0 / np.sqrt(d)
    o, _ = _forward(*(to_device(x, dtype) for x in (q, k, v)), form, scale)
    want = np.broadcast_to(synth.widen(v, dtype)[0, 0, 0], (B, H, Nq, d))
    assert_close_o(from_device(o), want, dtype, f"{form}/{dtype}/d{d} constant V")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_zero_queries_average_v(form, dtype):
    B, H, Nq, Nk, d = 2, 1, 64, 1000, 40
    q = synth.round_to(np.zeros((B, H, Nq, d)), dtype)
    k = synth.tensor(21, (B, H, Nk, d), dtype)
    v = synth.tensor(22, (B, H, Nk, d), dtype)
    o, ml = _forward(*(to_device(x, dtype) for x in (q, k, v)), form, 0.158)
    vd = synth.widen(v, dtype)
    want = np.broadcast_to(vd.mean(axis=2, keepdims=True), (B, H, Nq, d))
    assert_close_o(from_device(o), want, dtype, f"{form} q=0")
    mlh = from_device(ml)
    assert np.all(mlh[..., 0] == 0.0), "m of an all-zero score row must be 0"
    assert np.allclose(mlh[..., 1], Nk, rtol=1e-3), "l of an all-zero score row must be Nk"


@pytest.mark.parametrize("form", FORMS_O)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_key_shift_moves_m_only(form, dtype):
    # values on a 1/64 grid in [-2, 2] and a shift of 0.5: every value and sum
    # is a multiple of 1/64 below 4 in size, exact in fp16 and in bf16
    B, H, Nq, Nk, d = 1, 2, 96, 700, 40
    grid = lambda seed, n: np.round(np.clip(synth.normal(seed, n), -2, 2) * 64) / 64
    q = synth.round_to(grid(31, B * H * Nq * d).reshape(B, H, Nq, d), dtype)
    k = synth.round_to(grid(32, B * H * Nk * d).reshape(B, H, Nk, d), dtype)
    u = np.round(synth.uniform01(33, d) * 2 - 1) * 0.5
    k2 = synth.round_to(synth.widen(k, dtype) + u, dtype)
    assert np.array_equal(synth.widen(k2, dtype), synth.widen(k, dtype) + u)
    v = synth.tensor(34, (B, H, Nk, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    dev = lambda x: to_device(x, dtype)
    o1, ml1 = _forward(dev(q), dev(k), dev(v), form, scale)
    o2, ml2 = _forward(dev(q), dev(k2), dev(v), form, scale)
    o_ref, ml_ref = reference(q, k, v, dtype, scale)
    assert_close_o(from_device(o1), o_ref, dtype, f"{form} unshifted")
    assert_close_o(from_device(o2), o_ref, dtype, f"{form} shifted keys")
    shift = scale * (synth.widen(q, dtype) @ u)
    ml_ref2 = ml_ref.copy()
    ml_ref2[..., 0] += shift
    if ml1 is not None:
        assert_close_ml(from_device(ml1), ml_ref, f"{form} stats unshifted")
        assert_close_ml(from_device(ml2), ml_ref2, f"{form} stats shifted")


@pytest.mark.parametrize("form", FORMS_O)
@pytest.mark.parametrize("where", [0, 517, 4095])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dominant_key_takes_the_weight(form, where, dtype):
    B, H, Nq, Nk, d = 1, 1, 128, 4096, 40
    q = synth.tensor(41, (B, H, Nq, d), dtype, 0.5)
    k = synth.tensor(42, (B, H, Nk, d), dtype, 0.5)
    v = synth.tensor(43, (B, H, Nk, d), dtype)
    # the chosen key is a long vector along the mean query direction: for the
    # queries on its side it outweighs all other keys together
    qbar = synth.widen(q, dtype)[0, 0].mean(axis=0)
    k[0, 0, where] = synth.round_to(qbar / np.linalg.norm(qbar) * 200.0, dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, ml = _forward(*(to_device(x, dtype) for x in (q, k, v)), form, scale)
    o_ref, ml_ref = reference(q, k, v, dtype, scale)
    assert_close_o(from_device(o), o_ref, dtype, f"{form} dominant key at {where}")
    if ml is not None:
        assert_close_ml(from_device(ml), ml_ref, f"{form} dominant key at {where}")


@pytest.mark.parametrize("form", FORMS_O)
@pytest.mark.parametrize("dtype,d", [("f16", 40), ("bf16", 40), ("f16", 80), ("f16", 160)])
def test_rising_scores_rebase_every_block(form, dtype, d):
    # key j carries +j along the queries' mean direction: for the queries on
    # that side each 64-key block raises the row max by about 8 (in exp2
    # units), so the online state moves on nearly every block
    B, H, Nq, Nk = 1, 1, 160, 2100
    q = synth.tensor(51, (B, H, Nq, d), dtype, 0.5)
    qd = synth.widen(q, dtype)[0, 0]
    dirn = qd.mean(axis=0)
    dirn /= np.linalg.norm(dirn)
    kd = synth.normal(52, Nk * d).reshape(Nk, d) * 0.3 + np.arange(Nk)[:, None] * 1.0 * dirn
    k = synth.round_to(kd.reshape(B, H, Nk, d), dtype)
    v = synth.tensor(53, (B, H, Nk, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, ml = _forward(*(to_device(x, dtype) for x in (q, k, v)), form, scale)
    o_ref, ml_ref = reference(q, k, v, dtype, scale)
    assert_close_o(from_device(o), o_ref, dtype, f"{form}/{dtype}/d{d} rising scores")
    if ml is not None:
        assert_close_ml(from_device(ml), ml_ref, f"{form}/{dtype}/d{d} rising scores")


@pytest.mark.parametrize("gap", [15.5, 17.8, 19.5])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("form", ["flash", "flash_o"])
def test_late_key_within_the_fast_path_headroom(gap, dtype, form):
    # every query scores ~0 on every key but one late key, which scores `gap`
    # (exp2 units) above the first tile: beyond 16 the fp16 single pass keeps
    # P finite only through the 4 units of headroom of its reference max, with
    # P of that key up to 2^15.5 (no recompute of the pass)
    B, H, Nq, Nk, d = 1, 1, 64, 2048, 40
    scale = float(np.float32(1 / np.sqrt(d)))
    q = np.zeros((B, H, Nq, d))
    q[..., 0] = 1.0
    q[..., 1:] = synth.normal(71, Nq * (d - 1)).reshape(B, H, Nq, d - 1) * 0.05
    k = synth.normal(72, Nk * d).reshape(B, H, Nk, d) * 0.05
    k[0, 0, 1500, :] = 0.0
    k[0, 0, 1500, 0] = gap / (scale * np.log2(np.e))
    q, k = synth.round_to(q, dtype), synth.round_to(k, dtype)
    v = synth.tensor(73, (B, H, Nk, d), dtype)
    o, ml = _forward(*(to_device(x, dtype) for x in (q, k, v)), form, scale)
    o_ref, ml_ref = reference(q, k, v, dtype, scale)
    assert_close_o(from_device(o), o_ref, dtype, f"{form}: late key {gap} above the first tile")
    if ml is not None:
        assert_close_ml(from_device(ml), ml_ref, f"late key {gap} above the first tile")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("form", ["flash", "flash_o"])
def test_large_first_tile_reference_redoes_exactly(dtype, form):
    # the fp16 O-only single pass at head dim 40 folds the scale and a
    # reference of at most 64 (exp2 units) into the score product; rows
    # 0-63 here score ~80 and rows 64-95 ~300 on every key (dim 0 of the
    # query large, of every key ~1), so their workgroup redoes its rows on
    # the exact pass with the unscaled Q; the rows of the other workgroup
    # (ragged, 44 of 256) stay on the fast path
    B, H, Nq, Nk, d = 1, 2, 300, 1500, 40
    scale = float(np.float32(1 / np.sqrt(d)))
    c = scale * np.log2(np.e)
    q = synth.normal(81, B * H * Nq * d).reshape(B, H, Nq, d) * 0.5
    q[:, :, :64, 0] = 80.0 / c
    q[:, :, 64:96, 0] = 300.0 / c
    k = synth.normal(82, B * H * Nk * d).reshape(B, H, Nk, d) * 0.5
    k[..., 0] = 1.0 + 0.02 * synth.normal(83, B * H * Nk).reshape(B, H, Nk)
    q, k = synth.round_to(q, dtype), synth.round_to(k, dtype)
    v = synth.tensor(84, (B, H, Nk, d), dtype)
    o, ml = _forward(*(to_device(x, dtype) for x in (q, k, v)), form, scale)
    o_ref, ml_ref = reference(q, k, v, dtype, scale)
    assert_close_o(from_device(o), o_ref, dtype, f"{form}: large first-tile reference")
    if ml is not None:
        assert_close_ml(from_device(ml), ml_ref, f"{form}: large first-tile reference")


def test_scaled_query_overflow_redoes_exactly():
    # scale 2 and a query element of 60000: scaled into exp2 units (x 2.885)
    # it leaves fp16's range.  Keys 0-127 (the first tiles of both key
    # splits) have dim 0 = 0, so the reference stays near 0; keys from 128 on
    # have dim 0 = -2e-5 (an fp16 subnormal), true scores near -2.4, about
    # half of each row's weight, which an infinite scaled element would turn
    # into -inf scores and drop without any non-finite sum.  The overflow
    # itself sends the workgroup to the exact pass.  Half the queries carry
    # the large element.
    B, H, Nq, Nk, d, dtype, scale = 1, 1, 256, 1500, 40, "f16", 2.0
    q = synth.normal(91, B * H * Nq * d).reshape(B, H, Nq, d) * 0.1
    q[:, :, ::2, 0] = 60000.0
    k = synth.normal(92, B * H * Nk * d).reshape(B, H, Nk, d) * 0.1
    k[..., 0] = 0.0
    k[:, :, 128:, 0] = -2e-5
    q, k = synth.round_to(q, dtype), synth.round_to(k, dtype)
    v = synth.tensor(93, (B, H, Nk, d), dtype)
    o, _ = _forward(*(to_device(x, dtype) for x in (q, k, v)), "flash_o", scale)
    o_ref, _ = reference(q, k, v, dtype, scale)
    assert_close_o(from_device(o), o_ref, dtype, "scaled query beyond fp16")


@pytest.mark.parametrize("form", FORMS_O)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_peaked_softmax_large_logits(form, dtype):
    # Q, K ~ N(0, 3^2): scores spread over hundreds, most weights underflow
    cfg = CONFIGS["level2_self"]
    B, H, Nq, Nk, d = 1, 2, 256, 1024, 80
    q = synth.tensor(61, (B, H, Nq, d), dtype, 3.0)
    k = synth.tensor(62, (B, H, Nk, d), dtype, 3.0)
    v = synth.tensor(63, (B, H, Nk, d), dtype)
    o, ml = _forward(*(to_device(x, dtype) for x in (q, k, v)), form, cfg.scale)
    o_ref, ml_ref = reference(q, k, v, dtype, cfg.scale)
    assert_close_o(from_device(o), o_ref, dtype, f"{form} large logits")
    if ml is not None:
        assert_close_ml(from_device(ml), ml_ref, f"{form} large logits")


@pytest.mark.parametrize("name", ["sd512_cross", "level2_self"])
def test_bitwise_repeatable_and_stream_independent(name):
    import torch
    import attention_attn_stats_amd as attn
    cfg = CONFIGS[name]
    q, k, v = (to_device(x, cfg.dtype) for x in cfg.inputs())
    ref = {f: [t.clone() for t in _forward(q, k, v, f, cfg.scale)] for f in FORMS}
    ref["auto"] = [attn.forward(q, k, v, scale=cfg.scale)[0].clone()]
    for _ in range(3):
        for f in FORMS:
            got = _forward(q, k, v, f, cfg.scale)
            for a, b in zip(got, ref[f]):
                assert torch.equal(a, b), f"{name}/{f}: repeated launch differs"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = {f: _forward(q, k, v, f, cfg.scale) for f in FORMS}
        got_auto = attn.forward(q, k, v, scale=cfg.scale)[0]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for f in FORMS:
        for a, b in zip(got[f], ref[f]):
            assert torch.equal(a, b), f"{name}/{f}: side-stream result differs"
    assert torch.equal(got_auto, ref["auto"][0])


@pytest.mark.parametrize("d,qwg", [(40, 256), (80, 128), (160, 64)])
@pytest.mark.parametrize("form", FORMS + ("flash_o",))
@pytest.mark.parametrize("Nk", [300, 1000])
def test_workgroup_shape_does_not_change_results(d, qwg, form, Nk):
    """A problem with fewer workgroups than CUs runs with half the query groups
    per workgroup; each wave does the same work either way.  Row i depends on
    q_i, K and V only, so the first rows of a problem one workgroup short of
    filling the chip (halved shape) equal those of one that fills it (default
    shape) bit for bit.  At d = 80 the halved shape also cuts the keys into
    four splits of 32-key blocks instead of two: there the two agree to the
    rounding bound instead.  flash_o is the single pass without (m, l) out,
    whose fp16 form tests the rescale on the packed P."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    dtype = "f16"
    n_big = cus * qwg
    n_small = (cus - 1) * qwg
    q = synth.tensor(71 + d, (1, 1, n_big, d), dtype)
    k = synth.tensor(72 + d, (1, 1, Nk, d), dtype)
    v = synth.tensor(73 + d, (1, 1, Nk, d), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    tk, tv = to_device(k, dtype), to_device(v, dtype)

    def run(qh):
        if form == "flash_o":
            import attention_attn_stats_amd as attn
            return attn.flash(qh, tk, tv, scale=scale), None
        return _forward(qh, tk, tv, form, scale)

    o_big, ml_big = run(to_device(q, dtype))
    o_small, ml_small = run(to_device(np.ascontiguousarray(q[:, :, :n_small]), dtype))
    torch.cuda.synchronize()
    if d != 80:
        assert torch.equal(o_small, o_big[:, :, :n_small]), f"d={d} {form}: O differs between workgroup shapes"
        if ml_big is not None:
            assert torch.equal(ml_small, ml_big[:, :, :n_small])
    else:
        diff = (o_small.float() - o_big[:, :, :n_small].float()).abs().max().item()
        assert diff <= 2.0 ** -8, f"d={d} {form}: shapes differ by {diff}"
        if ml_big is not None:
            assert_close_ml(from_device(ml_small), from_device(ml_big[:, :, :n_small]), f"d={d} {form} shapes")
    for rows in (slice(0, 512), slice(n_small - 300, n_small)):
        o_ref, ml_ref = reference(q[:, :, rows], k, v, dtype, scale)
        assert_close_o(from_device(o_small)[:, :, rows], o_ref, dtype, f"d={d} {form} halved shape")
        if ml_small is not None:
            assert_close_ml(from_device(ml_small)[:, :, rows], ml_ref, f"d={d} {form} halved shape")
