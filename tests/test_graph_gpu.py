"""The kernels captured in a HIP graph (through torch.cuda.graph) and replayed:
every replay, with ordinary eager work and synchronisation between replays,
must reproduce the eager results bit for bit.  None of the entry points
records a memset or allocates inside the capture; the group-normalisation
workspace is sized and allocated by the first (eager) call.  A captured
group normalisation takes the two-launch form (the one-launch form's
call tags would repeat on every replay), so its eager reference is the
two-launch form too."""
import pytest

pytestmark = pytest.mark.gpu


def _inputs():
    import torch
    from attention_attn_stats_amd.configs import CONFIGS
    from gpu_util import to_device
    cfg = CONFIGS["sd512_cross"]
    q, k, v = (to_device(x, cfg.dtype) for x in cfg.inputs())
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((2, 320, 64 * 64), device="cuda", generator=g).half()
    h = torch.randn((2048, 2 * 1280), device="cuda", generator=g).half()
    return cfg, q, k, v, x, h


def _work(cfg, q, k, v, x, h, outs):
    import attention_attn_stats_amd as attn
    o_fl, ml_fl, o_pf, ml_pf, y, g = outs
    attn.flash(q, k, v, out=o_fl, ml=ml_fl, scale=cfg.scale)
    attn.stats(q, k, ml=ml_pf, scale=cfg.scale)
    attn.pv(q, k, v, ml_pf, out=o_pf, scale=cfg.scale)
    attn.group_norm(x, 32, eps=1e-5, out=y)
    attn.geglu(h, out=g)


def test_graph_replays_match_eager(monkeypatch):
    import torch
    cfg, q, k, v, x, h = _inputs()
    mk = lambda: [torch.empty_like(q), torch.empty((2, 8, cfg.Nq, 2), device="cuda"),
                  torch.empty_like(q), torch.empty((2, 8, cfg.Nq, 2), device="cuda"),
                  torch.empty_like(x), torch.empty((2048, 1280), device="cuda", dtype=torch.float16)]
    eager = mk()
    monkeypatch.setenv("ATTN_GN_PATH", "split")  # the form a captured call takes
    _work(cfg, q, k, v, x, h, eager)
    torch.cuda.synchronize()
    monkeypatch.delenv("ATTN_GN_PATH")
    outs = mk()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _work(cfg, q, k, v, x, h, outs)
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))  # ordinary eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager run"


def test_group_norm_graph_on_the_stream_of_earlier_calls():
    """A graph captured on a stream whose earlier eager group_norm calls
    allocated the workspace reuses it, unzeroed, on every replay; with new
    data in x before each replay, every replay must match the eager result
    for that data (the captured call must not mistake the previous replay's
    slice moments for its own)."""
    import torch
    import attention_attn_stats_amd as attn
    s = torch.cuda.Stream()
    g = torch.Generator(device="cuda").manual_seed(21)
    xs = [(torch.randn((2, 320, 64 * 64), device="cuda", generator=g) * (1 + i) + 0.5 * i).half()
          for i in range(3)]
    x, y = torch.empty_like(xs[0]), torch.empty_like(xs[0])
    with torch.cuda.stream(s):
        refs = [attn.group_norm(xi, 32, eps=1e-5) for xi in xs]
        x.copy_(xs[0])
        attn.group_norm(x, 32, eps=1e-5, out=y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        attn.group_norm(x, 32, eps=1e-5, out=y)
    for rep in range(6):
        i = rep % 3
        x.copy_(xs[i])
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        err = (y.float() - refs[i].float()).abs().max().item()
        assert err <= 8e-3, f"replay {rep} (data {i}): max difference {err} from the eager result"


def test_auto_forward_captured_for_an_untimed_shape():
    """ATTN_AUTO on a shape not yet timed, inside a capture: nothing may
    synchronise there, so the call takes the default variant (the two-pass
    form at d = 80) and the replay reproduces it bit for bit."""
    import torch
    import attention_attn_stats_amd as attn
    attn.select_reset()
    g = torch.Generator(device="cuda").manual_seed(22)
    q, k, v = (torch.randn((1, 2, 300, 80), device="cuda", generator=g).half() for _ in range(3))
    out = torch.empty_like(q)
    ml = torch.empty((1, 2, 300, 2), device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chosen = attn.select(1, 2, 300, 300, 80)  # no timing inside the capture either
        attn.forward(q, k, v, variant="auto", out=out, ml=ml)
    assert chosen == "pf"
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ml_ref = attn.stats(q, k)
    o_ref = attn.pv(q, k, v, ml_ref)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(ml, ml_ref)
    # the shape was not cached by the captured call: an eager call times it now
    o2, _ = attn.forward(q, k, v, variant="auto")
    torch.cuda.synchronize()
    assert (o2.float() - o_ref.float()).abs().max().item() <= 5e-3
