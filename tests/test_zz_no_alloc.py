"""The allocation-free group normalisation, attn_group_norm_static, against
attn_group_norm with a workspace the caller allocates: both run the same
kernels on the same plan, so their outputs must be bitwise equal.  Two calls
in a row on the library's fixed scratch, the second on a smaller problem,
through the C ABI; and a problem too large for the fixed scratch is refused
before launch."""
import ctypes

import pytest

pytestmark = pytest.mark.gpu

# (N, C, HW), groups: groups too large for one workgroup's registers, so the
# split forms (and their workspace) are used; the second problem is smaller
CASES = [((1, 128, 256 * 256), 32), ((1, 64, 200 * 200), 16)]


def _inputs(shape, dtype, seed):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    N, C, HW = shape
    x = (torch.randn((N, C, HW), device="cuda", dtype=torch.float32, generator=g) * 3 + 1).to(dtype)
    gamma = (torch.rand((C,), device="cuda", dtype=torch.float32, generator=g) + 0.5).to(dtype)
    beta = torch.randn((C,), device="cuda", dtype=torch.float32, generator=g).to(dtype)
    return x, gamma, beta


def _run_workspace(lib, x, gamma, beta, G, dt, stream):
    import torch
    N, C, HW = x.shape
    y = torch.empty_like(x)
    need = lib.attn_group_norm_workspace_size(x.data_ptr(), y.data_ptr(), N, C, HW, G, dt)
    assert need > 0, "the case must use the split forms"
    ws = torch.zeros(need, device="cuda", dtype=torch.uint8)
    st = lib.attn_group_norm(x.data_ptr(), gamma.data_ptr(), beta.data_ptr(), y.data_ptr(), ws.data_ptr(), need,
                             N, C, HW, G, 1e-5, dt, stream)
    assert st == 0, st
    return y


def _run_static(lib, x, gamma, beta, G, dt, stream):
    import torch
    N, C, HW = x.shape
    y = torch.empty_like(x)
    st = lib.attn_group_norm_static(x.data_ptr(), gamma.data_ptr(), beta.data_ptr(), y.data_ptr(), N, C, HW, G,
                                    1e-5, dt, stream)
    assert st == 0, st
    return y


@pytest.mark.parametrize("dtype_name", ["float16", "bfloat16", "float32"])
def test_static_scratch_matches_caller_workspace(dtype_name):
    import torch
    from attention_attn_stats_amd import _lib
    from attention_attn_stats_amd.api import _DT, _stream
    lib = _lib.load()
    dtype = getattr(torch, dtype_name)
    dt = _DT[dtype]
    for i, (shape, G) in enumerate(CASES):
        print(f"group_norm_static {dtype_name} {shape} G={G}", flush=True)
        x, gamma, beta = _inputs(shape, dtype, 100 + i)
        stream = _stream(x)
        ref = _run_workspace(lib, x, gamma, beta, G, dt, stream)
        got = _run_static(lib, x, gamma, beta, G, dt, stream)
        torch.cuda.synchronize()
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(got, ref), f"case {i}: max diff {(got.float() - ref.float()).abs().max().item()}"


def test_static_scratch_refuses_too_large_problem():
    import torch
    from attention_attn_stats_amd import _lib
    from attention_attn_stats_amd.api import _DT
    lib = _lib.load()
    x = torch.zeros(64, device="cuda", dtype=torch.float16)
    f = _DT[torch.float16]
    need = lib.attn_group_norm_workspace_size(x.data_ptr(), x.data_ptr(), 1024, 256, 65536, 32, f)
    assert need > 262144
    assert lib.attn_group_norm_static(x.data_ptr(), None, None, x.data_ptr(), 1024, 256, 65536, 32, 1e-5, f,
                                      None) == _lib.ERR_INVALID_ARG
