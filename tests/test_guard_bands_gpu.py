"""Guard bands around the dense outputs: out and ml (and the stored logit
matrix) are carved from the middle of larger buffers whose head and tail
hold a sentinel pattern; after every form runs on ragged shapes (query and key
counts that leave partial tiles, blocks and key splits), the outputs must match
the oracle and every sentinel must be intact (a kernel that writes past the
end of a row, a tile or a tensor -- for instance in the merge of key splits --
is caught here)."""
import numpy as np
import pytest

from attention_attn_stats_amd.configs import Config
from gpu_util import assert_close_ml, assert_close_o, from_device, reference, to_device

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes of sentinel before and after each output
SHAPES = [  # B, H, Nq, Nk, d
    (1, 1, 1, 1, 40), (1, 2, 77, 77, 40), (2, 1, 129, 63, 40), (1, 3, 300, 257, 40),
    (1, 2, 33, 31, 80), (2, 1, 100, 65, 80), (1, 1, 17, 33, 160), (1, 2, 140, 97, 160),
]


def _guarded(shape, torch_dtype):
    """A contiguous tensor of `shape` inside a byte buffer with GUARD sentinel
    bytes on each side (the tensor starts 16-byte aligned)."""
    import torch
    esz = torch.empty((), dtype=torch_dtype).element_size()
    n = int(np.prod(shape)) * esz
    buf = torch.full((GUARD + n + GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
    t = buf[GUARD:GUARD + n].view(torch_dtype).view(shape)
    return buf, t


def _intact(buf, n_bytes, what):
    head = buf[:GUARD]
    tail = buf[GUARD + n_bytes:]
    assert bool((head == 0xA5).all()), f"{what}: sentinel before the output overwritten"
    assert bool((tail == 0xA5).all()), f"{what}: sentinel after the output overwritten"


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_outputs_stay_inside_their_buffers(shape, dtype):
    import torch
    import attention_attn_stats_amd as attn
    B, H, Nq, Nk, d = shape
    cfg = Config(f"guard_{'x'.join(map(str, shape))}", 900 + sum(shape), B, H, Nq, Nk, d, dtype)
    q, k, v = cfg.inputs(dtype)
    o_ref, ml_ref = reference(q, k, v, dtype, cfg.scale)
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    osz = tq.numel() * tq.element_size()
    mlsz = B * H * Nq * 2 * 4

    def fresh():
        ob, o = _guarded((B, H, Nq, d), tq.dtype)
        mb, ml = _guarded((B, H, Nq, 2), torch.float32)
        return ob, o, mb, ml

    ob, o, mb, ml = fresh()
    attn.stats(tq, tk, ml=ml, scale=cfg.scale)
    attn.pv(tq, tk, tv, ml, out=o, scale=cfg.scale)
    torch.cuda.synchronize()
    _intact(mb, mlsz, "stats ml"), _intact(ob, osz, "pv out")
    assert_close_ml(from_device(ml), ml_ref, "stats")
    assert_close_o(from_device(o), o_ref, dtype, "pv")

    ob, o, mb, ml = fresh()
    attn.flash(tq, tk, tv, out=o, ml=ml, scale=cfg.scale)
    torch.cuda.synchronize()
    _intact(mb, mlsz, "flash ml"), _intact(ob, osz, "flash out")
    assert_close_ml(from_device(ml), ml_ref, "flash ml")
    assert_close_o(from_device(o), o_ref, dtype, "flash")

    ob, o, _, _ = fresh()
    attn.flash(tq, tk, tv, out=o, scale=cfg.scale)
    torch.cuda.synchronize()
    _intact(ob, osz, "flash (O only) out")
    assert_close_o(from_device(o), o_ref, dtype, "flash O only")

    for var in ("pf", "flash", "auto"):
        ob, o, mb, ml = fresh()
        attn.forward(tq, tk, tv, variant=var, out=o, ml=ml, scale=cfg.scale)
        torch.cuda.synchronize()
        _intact(mb, mlsz, f"forward {var} ml"), _intact(ob, osz, f"forward {var} out")
        assert_close_o(from_device(o), o_ref, dtype, f"forward {var}")

    if dtype != "f32":  # the stored-logit form runs on the matrix cores only
        ab, a = _guarded((B, H, Nq, Nk), torch.float32)
        ob, o, mb, ml = fresh()
        attn.scores(tq, tk, a=a, scale=cfg.scale)
        attn.scores_stats(a, ml=ml)
        attn.scores_pv(a, ml, tv, out=o)
        torch.cuda.synchronize()
        _intact(ab, B * H * Nq * Nk * 4, "scores a"), _intact(mb, mlsz, "scores_stats ml")
        _intact(ob, osz, "scores_pv out")
        assert_close_ml(from_device(ml), ml_ref, "scores_stats")
        assert_close_o(from_device(o), o_ref, dtype, "scores_pv")
