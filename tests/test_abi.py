"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/attn.h, and rejects bad arguments before touching the
device (no kernel is launched in these tests)."""
import ctypes
import os
import re

import pytest

from attention_attn_stats_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "attn.h")).read()
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libattn.so not built")
    return _lib.load()


def test_header_and_binding_agree():
    assert set(_declared()) == set(_lib.EXPORTS)


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++11")])
def test_header_is_plain_c_and_cxx(tmp_path, lang, std):
    # includable without HIP headers, from C and C++, warning-free; a C
    # program linking against the library resolves every entry point
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    src = tmp_path / ("use.c" if lang == "c" else "use.cpp")
    calls = "\n".join(f"  (void)&{n};" for n in _declared())
    src.write_text('#include "attn.h"\nint main(void) {\n' + calls + '\n  return attn_status_string(ATTN_OK) == 0;\n}\n')
    cmd = [cc, std, "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o",
           str(tmp_path / "use")]
    if os.path.exists(_lib.LIB_PATH):
        cmd += [_lib.LIB_PATH]
    else:
        cmd = cmd[:-2] + ["-fsyntax-only"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(4):
        assert lib.attn_status_string(s).decode()
    assert lib.attn_status_string(99).decode() == "unknown status"


def test_default_variant_follows_the_pages_rule(lib):
    assert lib.attn_default_variant(40) == _lib.FLASH
    assert lib.attn_default_variant(80) == _lib.PARTIAL_FUSED
    assert lib.attn_default_variant(160) == _lib.PARTIAL_FUSED


P = 1 << 20  # an aligned fake device address; never dereferenced: validation fails first


@pytest.mark.parametrize("args,expect", [
    # null pointers
    (dict(q=0), _lib.ERR_INVALID_ARG),
    (dict(k=0), _lib.ERR_INVALID_ARG),
    (dict(ml=0), _lib.ERR_INVALID_ARG),
    # misaligned pointers
    (dict(q=P + 8), _lib.ERR_INVALID_ARG),
    (dict(ml=P + 4), _lib.ERR_INVALID_ARG),
    # sizes
    (dict(B=0), _lib.ERR_INVALID_ARG),
    (dict(H=-1), _lib.ERR_INVALID_ARG),
    (dict(Nq=0), _lib.ERR_INVALID_ARG),
    (dict(Nk=0), _lib.ERR_INVALID_ARG),
    (dict(B=1 << 16, H=1 << 10, Nq=1 << 12), _lib.ERR_INVALID_ARG),
    # scale
    (dict(scale=float("nan")), _lib.ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.ERR_INVALID_ARG),
    (dict(scale=0.0), _lib.ERR_INVALID_ARG),
    (dict(scale=-0.5), _lib.ERR_INVALID_ARG),
    # unsupported head dim / dtype
    (dict(d=64), _lib.ERR_UNSUPPORTED),
    (dict(d=41), _lib.ERR_UNSUPPORTED),
    (dict(dt=7), _lib.ERR_UNSUPPORTED),
])
def test_stats_validation(lib, args, expect):
    a = dict(q=P, k=P, ml=P, B=1, H=1, Nq=8, Nk=8, d=40, scale=0.1, dt=_lib.F16)
    a.update(args)
    r = lib.attn_stats(a["q"] or None, a["k"] or None, a["ml"] or None, a["B"], a["H"], a["Nq"], a["Nk"],
                       a["d"], a["scale"], a["dt"], None)
    assert r == expect


def test_pv_flash_forward_validation(lib):
    f = _lib.F16
    assert lib.attn_pv(P, P, None, P, P, 1, 1, 8, 8, 40, 0.1, f, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_pv(P, P, P, None, P, 1, 1, 8, 8, 40, 0.1, f, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_flash(P, P, P, None, None, 1, 1, 8, 8, 40, 0.1, f, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_flash(P, P, P, P, None, 1, 1, 8, 8, 48, 0.1, f, None) == _lib.ERR_UNSUPPORTED
    # the partially fused form needs the (m, l) buffer
    assert lib.attn_forward(P, P, P, P, None, 1, 1, 8, 8, 40, 0.1, _lib.PARTIAL_FUSED, f, None) == \
        _lib.ERR_INVALID_ARG
    assert lib.attn_forward(P, P, P, P, P, 1, 1, 8, 8, 40, 0.1, 9, f, None) == _lib.ERR_UNSUPPORTED
    assert lib.attn_select(0, 1, 8, 8, 40, f, None) == _lib.AUTO


def test_scores_entry_points_validation(lib):
    f = _lib.F16
    # attn_scores: pointers, alignment, sizes, element type
    assert lib.attn_scores(None, P, P, 1, 1, 8, 8, 40, 0.1, f, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_scores(P, P, P + 2, 1, 1, 8, 8, 40, 0.1, f, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_scores(P, P, P, 1, 1, 8, 8, 64, 0.1, f, None) == _lib.ERR_UNSUPPORTED
    assert lib.attn_scores(P, P, P, 1, 1, 8, 8, 40, 0.1, _lib.F32, None) == _lib.ERR_UNSUPPORTED
    assert lib.attn_scores(P, P, P, 1, 1, 8, 8, 40, float("nan"), f, None) == _lib.ERR_INVALID_ARG
    # one head's A must stay below 2^31 bytes
    assert lib.attn_scores(P, P, P, 1, 1, 1 << 15, 1 << 14, 40, 0.1, f, None) == _lib.ERR_INVALID_ARG
    # attn_scores_stats
    assert lib.attn_scores_stats(None, P, 1, 1, 8, 8, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_scores_stats(P, P + 4, 1, 1, 8, 8, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_scores_stats(P, P, 1, 1, 8, 0, None) == _lib.ERR_INVALID_ARG
    # attn_scores_pv
    assert lib.attn_scores_pv(P, P, None, P, 1, 1, 8, 8, 40, f, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_scores_pv(P, P, P, P + 8, 1, 1, 8, 8, 40, f, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_scores_pv(P, P, P, P, 1, 1, 8, 8, 80, _lib.F32, None) == _lib.ERR_UNSUPPORTED
    assert lib.attn_scores_pv(P, P, P, P, 1, 1, 8, 8, 48, f, None) == _lib.ERR_UNSUPPORTED


def _layout(row_q=40, row_k=40, row_v=40, row_o=40, head=0, batch=0):
    S = _lib.Strides
    return _lib.Layout(S(batch, head, row_q), S(batch, head, row_k), S(batch, head, row_v), S(batch, head, row_o))


@pytest.mark.parametrize("lay", [
    _layout(row_q=32),                 # row shorter than d
    _layout(row_k=44),                 # row stride not a multiple of 16 bytes
    _layout(head=-8),                  # negative stride
    _layout(batch=4),                  # batch stride not a multiple of 16 bytes
    _layout(row_v=1 << 27),            # one head's rows span more than 2^30 elements
    _layout(row_o=36),                 # the output is checked too
    _layout(row_k=(1 << 20) + 8),      # row stride past 2^20 elements (64-row blocks use 32-bit offsets)
])
def test_strided_layout_validation(lib, lay):
    f = _lib.F16
    r = ctypes.byref(lay)
    assert lib.attn_flash_strided(P, P, P, P, None, r, 1, 1, 16, 16, 40, 0.1, f, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_forward_strided(P, P, P, P, P, r, 1, 1, 16, 16, 40, 0.1, _lib.AUTO, f, None) == \
        _lib.ERR_INVALID_ARG
    assert lib.attn_pv_strided(P, P, P, P, P, r, 1, 1, 16, 16, 40, 0.1, f, None) == _lib.ERR_INVALID_ARG


def test_strided_stats_checks_only_q_and_k(lib):
    f = _lib.F16
    bad_q = _lib.Layout(_lib.Strides(0, 0, 36), _lib.Strides(0, 0, 40), _lib.Strides(), _lib.Strides())
    assert lib.attn_stats_strided(P, P, P, ctypes.byref(bad_q), 1, 1, 8, 8, 40, 0.1, f, None) == \
        _lib.ERR_INVALID_ARG
    # f32 rows need 4-element (16-byte) multiples only
    bad_f32 = _layout(row_q=42)
    assert lib.attn_stats_strided(P, P, P, ctypes.byref(bad_f32), 1, 1, 8, 8, 40, 0.1, _lib.F32, None) == \
        _lib.ERR_INVALID_ARG
    # the plain checks still come first
    assert lib.attn_stats_strided(None, P, P, None, 1, 1, 8, 8, 40, 0.1, f, None) == _lib.ERR_INVALID_ARG
    assert lib.attn_stats_strided(P, P, P, None, 1, 1, 8, 8, 64, 0.1, f, None) == _lib.ERR_UNSUPPORTED


def test_group_norm_and_geglu_validation(lib):
    f = _lib.F16
    # attn_group_norm(x, gamma, beta, y, workspace, workspace_bytes, N, C, HW, G, eps, dt, stream)
    def gn(x, ga, be, y, ws, N, C, HW, G, eps, dt):
        return lib.attn_group_norm(x, ga, be, y, ws, 1 << 20, N, C, HW, G, eps, dt, None)
    assert gn(None, None, None, P, P, 2, 32, 64, 32, 1e-5, f) == _lib.ERR_INVALID_ARG
    assert gn(P, None, None, None, P, 2, 32, 64, 32, 1e-5, f) == _lib.ERR_INVALID_ARG
    assert gn(P, None, None, P, P, 2, 30, 64, 4, 1e-5, f) == _lib.ERR_INVALID_ARG      # C % G
    assert gn(P, None, None, P, P, 0, 32, 64, 32, 1e-5, f) == _lib.ERR_INVALID_ARG     # N
    assert gn(P, None, None, P, P, 2, 32, 0, 32, 1e-5, f) == _lib.ERR_INVALID_ARG      # HW
    assert gn(P, None, None, P, P, 2, 32, 64, 0, 1e-5, f) == _lib.ERR_INVALID_ARG      # G
    assert gn(P, None, None, P, P, 2, 32, 64, 32, -1.0, f) == _lib.ERR_INVALID_ARG     # eps
    assert gn(P, None, None, P, P, 2, 32, 64, 32, float("nan"), f) == _lib.ERR_INVALID_ARG
    assert gn(P + 1, None, None, P, P, 2, 32, 64, 32, 1e-5, f) == _lib.ERR_INVALID_ARG  # x alignment
    assert gn(P, P + 1, None, P, P, 2, 32, 64, 32, 1e-5, f) == _lib.ERR_INVALID_ARG     # gamma alignment
    assert gn(P, None, None, P, P + 4, 2, 32, 64, 32, 1e-5, f) == _lib.ERR_INVALID_ARG  # workspace alignment
    assert gn(P + 2, None, None, P, P, 2, 32, 64, 32, 1e-5, _lib.F32) == _lib.ERR_INVALID_ARG
    assert gn(P, None, None, P, P, 1 << 16, 1 << 12, 1 << 12, 32, 1e-5, f) == _lib.ERR_INVALID_ARG
    assert gn(P, None, None, P, P, 2, 32, 64, 32, 1e-5, 9) == _lib.ERR_UNSUPPORTED
    # workspace: none for groups that fit one workgroup, some for larger ones,
    # and a missing or short one is refused before launch
    ws = lib.attn_group_norm_workspace_size
    assert ws(P, P, 2, 2560, 8 * 8, 32, f) == 0       # small groups: one launch
    assert ws(P, P, 8, 320, 64 * 64, 32, f) == 0      # 256 groups fill the chip: one launch
    need = ws(P, P, 2, 640, 128 * 128, 32, f)
    assert need > 0 and need % 8 == 0
    assert ws(P, P, 2, 30, 64, 4, f) == 0  # invalid sizes
    assert lib.attn_group_norm(P, None, None, P, None, 0, 2, 640, 128 * 128, 32, 1e-5, f, None) == \
        _lib.ERR_INVALID_ARG
    assert lib.attn_group_norm(P, None, None, P, P, need - 8, 2, 640, 128 * 128, 32, 1e-5, f, None) == \
        _lib.ERR_INVALID_ARG
    # attn_group_norm_static: the same argument checks, and a problem whose
    # workspace exceeds the fixed 262144 bytes is refused before launch
    st = lib.attn_group_norm_static
    assert st(None, None, None, P, 2, 32, 64, 32, 1e-5, f, None) == _lib.ERR_INVALID_ARG
    assert st(P, None, None, None, 2, 32, 64, 32, 1e-5, f, None) == _lib.ERR_INVALID_ARG
    assert st(P, None, None, P, 2, 30, 64, 4, 1e-5, f, None) == _lib.ERR_INVALID_ARG
    assert st(P, None, None, P, 2, 32, 64, 32, -1.0, f, None) == _lib.ERR_INVALID_ARG
    assert st(P, None, None, P, 2, 32, 64, 32, 1e-5, 9, None) == _lib.ERR_UNSUPPORTED
    big = ws(P, P, 1024, 256, 65536, 32, f)
    assert big > 262144
    assert st(P, None, None, P, 1024, 256, 65536, 32, 1e-5, f, None) == _lib.ERR_INVALID_ARG
    # attn_geglu(h, out, rows, F, dt, stream)
    ge = lib.attn_geglu
    assert ge(None, P, 4, 8, f, None) == _lib.ERR_INVALID_ARG
    assert ge(P, None, 4, 8, f, None) == _lib.ERR_INVALID_ARG
    assert ge(P, P, 0, 8, f, None) == _lib.ERR_INVALID_ARG
    assert ge(P, P, 4, 0, f, None) == _lib.ERR_INVALID_ARG
    assert ge(P + 1, P, 4, 8, f, None) == _lib.ERR_INVALID_ARG
    assert ge(P, P, 1 << 16, 1 << 15, f, None) == _lib.ERR_INVALID_ARG  # rows * F >= 2^31 - 512
    assert ge(P, P, 4, 8, 9, None) == _lib.ERR_UNSUPPORTED


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no fallback: without libattn.so every entry point raises, naming the
    # build command
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libattn.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError, match="attention_attn_stats_amd.build"):
        _lib.load()
