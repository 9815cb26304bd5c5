"""Python entry points with the same names as the C ABI (include/attn.h).

Argument marshalling only: shapes and element types are checked, pointers and
the current HIP stream are handed to libattn.so, and any non-OK status is
raised as AttnError.  Nothing here computes attention.

q, k, v and out may be strided views (for example the [B, N, H*d] activations
of a transformer block viewed as [B, H, N, d] with
``x.view(B, N, H, d).transpose(1, 2)``) as long as the last dimension is
contiguous; such calls go through the *_strided entry points with the
tensors' own strides, without a copy.
"""
from __future__ import annotations

import collections
import math

import torch

from . import _lib
from ._lib import AttnError

_DT = {torch.float32: _lib.F32, torch.float16: _lib.F16, torch.bfloat16: _lib.BF16}
_VAR = {"auto": _lib.AUTO, "pf": _lib.PARTIAL_FUSED, "partial_fused": _lib.PARTIAL_FUSED,
        "flash": _lib.FLASH}
_VAR_NAME = {_lib.AUTO: "auto", _lib.PARTIAL_FUSED: "pf", _lib.FLASH: "flash"}


def _check(status: int, where: str):
    if status != _lib.OK:
        raise AttnError(status, where)


def _dims(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor | None):
    # (every attribute read costs a fraction of a microsecond: each is read once)
    qs, ks = q.shape, k.shape
    if len(qs) != 4 or len(ks) != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, H, Nq, d = qs
    Bk, Hk, Nk, dk = ks
    if Bk != B or Hk != H or dk != d:
        raise ValueError(f"k shape {tuple(ks)} does not match q {tuple(qs)}")
    if v is not None and v.shape != ks:
        raise ValueError(f"v shape {tuple(v.shape)} must equal k shape {tuple(ks)}")
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    dev = q.device
    for t in (q, k, v):
        if t is not None and (not t.is_cuda or t.dtype != dt or (d > 1 and t.stride(3) != 1) or t.device != dev):
            raise ValueError("q, k, v must be tensors on one device, of one dtype, with contiguous rows")
    return B, H, Nq, Nk, d


def _check_ml(ml, shape, device):
    if (ml.shape != shape or ml.dtype != torch.float32 or not ml.is_contiguous() or not ml.is_cuda
            or ml.device != device):
        raise ValueError(f"ml must be a contiguous float32 {list(shape)} tensor on {device}")


def _strides(t: torch.Tensor) -> _lib.Strides:
    # the stride of a dimension of extent 1 is never used; torch may report
    # any value there, so pass one that satisfies the library's checks
    b, h, n, d = t.shape
    return _lib.Strides(t.stride(0) if b > 1 else 0, t.stride(1) if h > 1 else 0,
                        t.stride(2) if n > 1 else d)


def _layout(q, k, v=None, out=None):
    """None when every tensor is dense (the plain entry points), else the
    attn_layout of their strides."""
    if (q.is_contiguous() and k.is_contiguous() and (v is None or v.is_contiguous())
            and (out is None or out.is_contiguous())):
        return None
    z = _lib.Strides(0, 0, 0)
    return _lib.Layout(_strides(q), _strides(k), _strides(v) if v is not None else z,
                       _strides(out) if out is not None else z)


def _out_for(q, out):
    if out is None:
        return torch.empty_like(q)  # keeps q's strides when q is a dense view
    if (out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda or out.stride(3) != 1
            or out.device != q.device):
        raise ValueError("out must be a tensor on q's device, of q's shape and dtype, with contiguous rows")
    # (a contiguous tensor cannot overlap itself)
    if not out.is_contiguous() and torch._debug_has_internal_overlap(out) == 1:
        raise ValueError("out must not have overlapping elements")
    return out


def _scale(scale, d):
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor | None = None):
    """The current stream of t's device (else of the current device) as the
    handle the library takes; read without building a torch Stream object
    where torch offers that."""
    dev = t.get_device() if t is not None else torch.cuda.current_device()
    if _raw_stream is not None:
        return _raw_stream(dev)
    return ctypes_stream(torch.cuda.current_stream(dev))


def ctypes_stream(s: torch.cuda.Stream):
    return s.cuda_stream


def _ml_for(q, ml):
    B, H, Nq, _ = q.shape
    if ml is None:
        return torch.empty((B, H, Nq, 2), device=q.device, dtype=torch.float32)
    _check_ml(ml, (B, H, Nq, 2), q.device)
    return ml


def stats(q, k, ml=None, scale=None):
    """Row statistics (m, l) of A = scale q k^T -> ml [B, H, Nq, 2] float32."""
    B, H, Nq, Nk, d = _dims(q, k, None)
    ml = _ml_for(q, ml)
    lay = _layout(q, k)
    args = (B, H, Nq, Nk, d, _scale(scale, d), _DT[q.dtype], _stream(q))
    if lay is None:
        _check(_lib.load().attn_stats(q.data_ptr(), k.data_ptr(), ml.data_ptr(), *args), "attn_stats")
    else:
        _check(_lib.load().attn_stats_strided(q.data_ptr(), k.data_ptr(), ml.data_ptr(), lay, *args),
               "attn_stats_strided")
    return ml


def pv(q, k, v, ml, out=None, scale=None):
    """O = softmax(A) v from statistics produced by stats()."""
    B, H, Nq, Nk, d = _dims(q, k, v)
    _check_ml(ml, (B, H, Nq, 2), q.device)
    out = _out_for(q, out)
    lay = _layout(q, k, v, out)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), ml.data_ptr(), out.data_ptr())
    args = (B, H, Nq, Nk, d, _scale(scale, d), _DT[q.dtype], _stream(q))
    if lay is None:
        _check(_lib.load().attn_pv(*ptrs, *args), "attn_pv")
    else:
        _check(_lib.load().attn_pv_strided(*ptrs, lay, *args), "attn_pv_strided")
    return out


def flash(q, k, v, out=None, ml=None, want_ml=False, scale=None):
    """Single-pass online-softmax attention.  Returns out, or (out, ml) if
    want_ml or ml is given."""
    B, H, Nq, Nk, d = _dims(q, k, v)
    out = _out_for(q, out)
    if want_ml or ml is not None:
        ml = _ml_for(q, ml)
    lay = _layout(q, k, v, out)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), ml.data_ptr() if ml is not None else None)
    args = (B, H, Nq, Nk, d, _scale(scale, d), _DT[q.dtype], _stream(q))
    if lay is None:
        _check(_lib.load().attn_flash(*ptrs, *args), "attn_flash")
    else:
        _check(_lib.load().attn_flash_strided(*ptrs, lay, *args), "attn_flash_strided")
    return (out, ml) if ml is not None else out


def forward(q, k, v, variant="auto", out=None, ml=None, scale=None):
    """Attention with the given variant ('auto', 'pf', 'flash'); returns (out, ml).
    ml holds the row statistics when the partially fused form ran and is
    untouched scratch when the single pass ran (use flash(..., want_ml=True))."""
    B, H, Nq, Nk, d = _dims(q, k, v)
    out = _out_for(q, out)
    ml = _ml_for(q, ml)
    lay = _layout(q, k, v, out)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), ml.data_ptr())
    args = (B, H, Nq, Nk, d, _scale(scale, d), _VAR[variant], _DT[q.dtype], _stream(q))
    if lay is None:
        _check(_lib.load().attn_forward(*ptrs, *args), "attn_forward")
    else:
        _check(_lib.load().attn_forward_strided(*ptrs, lay, *args), "attn_forward_strided")
    return out, ml


def _a_for(B, H, Nq, Nk, device, a):
    if a is None:
        return torch.empty((B, H, Nq, Nk), device=device, dtype=torch.float32)
    if (a.shape != (B, H, Nq, Nk) or a.dtype != torch.float32 or not a.is_contiguous() or not a.is_cuda
            or a.device != device):
        raise ValueError(f"a must be a contiguous float32 [B, H, Nq, Nk] tensor on {device}")
    return a


def scores(q, k, a=None, scale=None):
    """The stored logit matrix A = scale q k^T -> a [B, H, Nq, Nk] float32."""
    B, H, Nq, Nk, d = _dims(q, k, None)
    if not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("scores() takes contiguous q and k")
    a = _a_for(B, H, Nq, Nk, q.device, a)
    _check(_lib.load().attn_scores(q.data_ptr(), k.data_ptr(), a.data_ptr(), B, H, Nq, Nk, d,
                                   _scale(scale, d), _DT[q.dtype], _stream(q)), "attn_scores")
    return a


def scores_stats(a, ml=None):
    """Row statistics (m, l) of a stored A -> ml [B, H, Nq, 2] float32."""
    if a.dim() != 4 or a.dtype != torch.float32 or not a.is_cuda or not a.is_contiguous():
        raise ValueError("a must be a contiguous float32 [B, H, Nq, Nk] device tensor")
    B, H, Nq, Nk = a.shape
    if ml is None:
        ml = torch.empty((B, H, Nq, 2), device=a.device, dtype=torch.float32)
    else:
        _check_ml(ml, (B, H, Nq, 2), a.device)
    _check(_lib.load().attn_scores_stats(a.data_ptr(), ml.data_ptr(), B, H, Nq, Nk, _stream(a)),
           "attn_scores_stats")
    return ml


def scores_pv(a, ml, v, out=None):
    """O = softmax(A) v from a stored A and its statistics -> out [B, H, Nq, d]."""
    if a.dim() != 4 or a.dtype != torch.float32 or not a.is_cuda or not a.is_contiguous():
        raise ValueError("a must be a contiguous float32 [B, H, Nq, Nk] device tensor")
    B, H, Nq, Nk = a.shape
    if (v.dim() != 4 or tuple(v.shape[:3]) != (B, H, Nk) or not v.is_cuda or not v.is_contiguous()
            or v.device != a.device):
        raise ValueError(f"v {tuple(v.shape)} must be a contiguous tensor on a's device matching a {tuple(a.shape)}")
    if v.dtype not in _DT:
        raise ValueError(f"unsupported dtype {v.dtype}")
    _check_ml(ml, (B, H, Nq, 2), a.device)
    d = v.shape[3]
    out = torch.empty((B, H, Nq, d), device=v.device, dtype=v.dtype) if out is None else out
    if (out.shape != (B, H, Nq, d) or out.dtype != v.dtype or not out.is_contiguous() or not out.is_cuda
            or out.device != a.device):
        raise ValueError("out must be a contiguous [B, H, Nq, d] tensor of v's dtype on a's device")
    _check(_lib.load().attn_scores_pv(a.data_ptr(), ml.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, Nq, Nk,
                                      d, _DT[v.dtype], _stream(a)), "attn_scores_pv")
    return out


_GN_WS: "collections.OrderedDict" = collections.OrderedDict()
_GN_WS_MAX = 16  # streams with a cached workspace (least recently used dropped first)


def _gn_workspace(device, nbytes: int) -> torch.Tensor:
    """A group-normalisation workspace of at least nbytes, one per device and
    stream (kernels on one stream never overlap, so they may share it).  A
    workspace is allocated while its stream is current and used on that
    stream only, so dropping it from the cache is ordered after its last use
    by the allocator."""
    key = (device, _raw_stream(device.index) if _raw_stream is not None
           else torch.cuda.current_stream(device).cuda_stream)
    ws = _GN_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)  # zero-filled before first use
        _GN_WS[key] = ws
        while len(_GN_WS) > _GN_WS_MAX:
            _GN_WS.popitem(last=False)
    _GN_WS.move_to_end(key)
    return ws


def group_norm(x, groups: int, gamma=None, beta=None, eps: float = 1e-5, out=None):
    """Group normalisation of x [N, C, *spatial] (contiguous) with `groups`
    groups of consecutive channels -> y of x's shape and dtype.  gamma, beta:
    [C] in x's dtype or None.  out may be x (in place)."""
    if x.dim() < 2 or not x.is_cuda or not x.is_contiguous() or x.dtype not in _DT:
        raise ValueError("x must be a contiguous [N, C, ...] device tensor of a supported dtype")
    N, C = x.shape[:2]
    HW = x.numel() // (N * C) if N * C else 0
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None and (t.shape != (C,) or t.dtype != x.dtype or not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [C] device tensor of x's dtype")
    out = torch.empty_like(x) if out is None else out
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous device tensor of x's shape and dtype")
    lib = _lib.load()
    need = lib.attn_group_norm_workspace_size(x.data_ptr(), out.data_ptr(), N, C, HW, int(groups), _DT[x.dtype])
    ws = _gn_workspace(x.device, need) if need else None
    _check(lib.attn_group_norm(x.data_ptr(), gamma.data_ptr() if gamma is not None else None,
                               beta.data_ptr() if beta is not None else None, out.data_ptr(),
                               ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
                               N, C, HW, int(groups), float(eps), _DT[x.dtype], _stream(x)), "attn_group_norm")
    return out


def geglu(h, out=None):
    """GELU-gated product of h [..., 2F] (contiguous): h[..., :F] * gelu(h[..., F:])."""
    if h.dim() < 1 or not h.is_cuda or not h.is_contiguous() or h.dtype not in _DT or h.shape[-1] % 2:
        raise ValueError("h must be a contiguous device tensor of a supported dtype with an even last dim")
    F = h.shape[-1] // 2
    rows = h.numel() // (2 * F) if F else 0
    shape = tuple(h.shape[:-1]) + (F,)
    out = torch.empty(shape, device=h.device, dtype=h.dtype) if out is None else out
    if tuple(out.shape) != shape or out.dtype != h.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous device tensor [..., F] of h's dtype")
    _check(_lib.load().attn_geglu(h.data_ptr(), out.data_ptr(), rows, F, _DT[h.dtype], _stream(h)), "attn_geglu")
    return out


def select(B, H, Nq, Nk, d, dtype=torch.float16) -> str:
    """The variant 'auto' uses for this shape ('pf' or 'flash'); may time both."""
    r = _lib.load().attn_select(B, H, Nq, Nk, d, _DT[dtype], _stream())
    if r == _lib.AUTO:
        raise AttnError(_lib.ERR_HIP, "attn_select")
    return _VAR_NAME[r]


def select_reset():
    _lib.load().attn_select_reset()


def default_variant(d: int) -> str:
    return _VAR_NAME[_lib.load().attn_default_variant(int(d))]
