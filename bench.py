#!/usr/bin/env python3
"""Throughput of the SD UNet attention hot path on one MI355X.

One step = the attention forward over the seeded synthetic inputs of the SD
512x512 top-level self-attention (B=2, H=8, Nq=Nk=4096, d=40, fp16), inputs
already resident in HBM, in the form the per-shape selector picks (attn_select,
as attn_forward with ATTN_AUTO would), issued kernel by kernel as attn_forward
issues it: attn_flash for the single pass, or attn_stats then attn_pv for the
partially fused form.  With --variant the form is fixed instead.

Prints ONE JSON line with the headline metric (useful attention TFLOP/s,
4*B*H*Nq*Nk*d per step, and its fraction of the fp16 dense MFMA peak), the
roofline record of the dominant kernel (HIP-event durations of that kernel's
launches inside the timed region), and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                    [--variant auto|pf|flash] [--no-cpu-baseline]
                    [--configs-out FILE]   # also time every config and form, JSONL there
                    [--cold]               # configs table: evict the caches between steps
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s + % fp16 MFMA peak @ B=2,H=8,N=4096,d=40"
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}  # dense MFMA (fp16/bf16); fp32 vector
HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "attention_attn_stats_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source(kernel: str, cfg, cus: int = 256) -> str:
    """Source file of the kernel a launch runs, by the library's dispatch rule:
    in the half types, the single pass takes the short-key-range kernel of
    attn_short.hip where Nk <= 384 (d = 40) or 256 (d = 80, 160) (ATTN_SHORT=0
    / 1 turn that off / force it within those limits); otherwise the single
    pass and the second pass at d = 40 take the kernels of attn_fa40.hip when
    Nk > 1024 (ATTN_FA40=0 / 1 turn that off / force it); the
    general kernels of attn_mfma.hip take the rest."""
    half = cfg.dtype in ("f16", "bf16")
    short_max = {40: 384, 80: 256, 160: 256}.get(cfg.d, 0)
    env_s = os.environ.get("ATTN_SHORT", "")[:1]
    if half and kernel == "attn_flash" and cfg.Nk <= short_max and env_s != "0":
        return os.path.join(CSRC, "attn_short.hip")
    env = os.environ.get("ATTN_FA40", "")[:1]
    rule = cfg.Nk > 1024
    on = {"0": False, "1": True}.get(env, rule)
    fa40 = cfg.d == 40 and half and kernel in ("attn_flash", "attn_pv") and on
    return os.path.join(CSRC, "attn_fa40.hip" if fa40 else "attn_mfma.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(path: str) -> str:
    """Hash of a kernel source without its comments and blank space, and of
    the compile flags of that file alone, so that a comment edit does not
    orphan counters taken on the same code but a flag that changes the code
    does."""
    import re
    from attention_attn_stats_amd import build as _build
    with open(path) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = "\n".join(ln.strip() for ln in src.splitlines() if ln.strip())
    flags = _build.FILE_FLAGS.get(os.path.basename(path), [])
    if flags:
        src += "\n#flags " + " ".join(flags)
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def load_traffic(kernel: str, cfg):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on the current source of the kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(f"{kernel}@{cfg.name}")
    if not e or e.get("kernel_src_sha256_16") != kernel_hash(kernel_source(kernel, cfg)):
        return None
    return e.get("bytes_per_launch")


def device_inputs(cfg, layout: str = "bhnd"):
    """q, k, v on the device: dense [B, H, N, d], or (layout 'bnhd') [B, H, N, d]
    views of [B, N, H*d] tensors, the layout a UNet block's projections give."""
    import torch
    q, k, v = cfg.inputs()
    conv = {"f16": lambda a: torch.from_numpy(a), "f32": lambda a: torch.from_numpy(a),
            "bf16": lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16)}[cfg.dtype]
    if layout == "bnhd":
        return [conv(x.transpose(0, 2, 1, 3).copy()).cuda().transpose(1, 2) for x in (q, k, v)]
    return [conv(x).cuda().contiguous() for x in (q, k, v)]


def time_config(cfg, variant: str, steps: int, warmup: int):
    """Time `steps` forwards; returns a dict with per-step and per-kernel times."""
    import torch
    import attention_attn_stats_amd as attn
    q, k, v = device_inputs(cfg)
    out = torch.empty_like(q)
    ml = torch.empty((cfg.B, cfg.H, cfg.Nq, 2), device=q.device, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    # the selector decides (and caches) on the first call; the chosen form is
    # then issued kernel by kernel, as attn_forward issues it
    attn.forward(q, k, v, variant=variant, out=out, ml=ml, scale=cfg.scale)
    chosen = variant if variant != "auto" else attn.select(cfg.B, cfg.H, cfg.Nq, cfg.Nk, cfg.d,
                                                           q.dtype)

    def step(evs=None):
        if chosen == "flash":
            attn.flash(q, k, v, out=out, scale=cfg.scale)  # as attn_forward issues it: no statistics
        else:
            if evs:
                evs[0].record(stream)
            attn.stats(q, k, ml=ml, scale=cfg.scale)
            if evs:
                evs[1].record(stream)
            attn.pv(q, k, v, ml, out=out, scale=cfg.scale)
            if evs:
                evs[2].record(stream)

    for _ in range(warmup):
        step()
    # flash is one kernel per step: events bracket the whole timed region and
    # the launch average is its span / steps (the launches run back to back,
    # as in a network).  The two-kernel form records events around each kernel.
    evs = None if chosen == "flash" else [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                                          for _ in range(steps)]
    span = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    span[0].record(stream)
    for i in range(steps):
        step(evs[i] if evs else None)
    span[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = {}
    if chosen == "flash":
        kern["flash"] = span[0].elapsed_time(span[1]) / steps
    else:
        kern["stats"] = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        kern["pv"] = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    return {"variant": chosen, "ms_per_step": wall * 1e3 / steps, "kernel_ms": kern}


def algorithmic_bytes(cfg, form: str) -> dict:
    """HBM bytes each form must move at least once (element size from dtype);
    the '_bnhd' forms move the same bytes as their dense forms."""
    es = {"f16": 2, "bf16": 2, "f32": 4}[cfg.dtype]
    bh = cfg.B * cfg.H
    q, kv, ml = bh * cfg.Nq * cfg.d * es, bh * cfg.Nk * cfg.d * es, bh * cfg.Nq * 8
    stats = q + kv + ml                     # pass 1: read Q, K; write ml
    pv = q + 2 * kv + ml + q                # pass 2: read Q, K, V, ml; write O
    a = bh * cfg.Nq * cfg.Nk * 4            # the stored logit matrix (float32)
    sc = {"scores": q + kv + a, "scores_stats": a + ml, "scores_pv": a + ml + kv + q}
    r = {"flash": q + 2 * kv + q, "pf": stats + pv, "stats": stats,
         "pf_scores": sum(sc.values()), **sc}
    r.update({f"{f}_bnhd": r[f] for f in ("flash", "pf", "stats")})
    return r


def time_steps(cfg, form: str, steps: int, warmup: int, cold: bool):
    """Per-step times (ms) with events around every step, for the median / min
    of the configs table.  `cold` rewrites a 512 MiB buffer before every step
    (outside the events) so that K and V come from HBM, not L2 / MALL.  A form
    ending in '_bnhd' runs on [B, N, H*d] inputs and output (strided views)."""
    import statistics
    import torch
    import attention_attn_stats_amd as attn
    layout = "bnhd" if form.endswith("_bnhd") else "bhnd"
    form = form[:-len("_bnhd")] if layout == "bnhd" else form
    q, k, v = device_inputs(cfg, layout)
    out = torch.empty_like(q)
    ml = torch.empty((cfg.B, cfg.H, cfg.Nq, 2), device=q.device, dtype=torch.float32)
    a = (torch.empty((cfg.B, cfg.H, cfg.Nq, cfg.Nk), device=q.device, dtype=torch.float32)
         if form == "pf_scores" else None)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=q.device) if cold else None
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(warmup + steps):
        if scrub is not None:
            scrub.fill_(i & 0xFF)
        e = ev[i - warmup] if i >= warmup else None
        if e:
            e[0].record(stream)
        if form == "flash":
            attn.flash(q, k, v, out=out, scale=cfg.scale)
            if e:
                e[1].record(stream)
        elif form == "pf_scores":
            attn.scores(q, k, a, scale=cfg.scale)
            if e:
                e[1].record(stream)
            attn.scores_stats(a, ml)
            if e:
                e[3].record(stream)
            attn.scores_pv(a, ml, v, out=out)
        else:
            attn.stats(q, k, ml=ml, scale=cfg.scale)
            if e:
                e[1].record(stream)
            attn.pv(q, k, v, ml, out=out, scale=cfg.scale)
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    step = [e[0].elapsed_time(e[2]) for e in ev]
    first = [e[0].elapsed_time(e[1]) for e in ev]
    r = {"median_ms": statistics.median(step), "min_ms": min(step),
         "first_kernel_median_ms": statistics.median(first)}
    if form == "pf_scores":
        r["second_kernel_median_ms"] = statistics.median([e[1].elapsed_time(e[3]) for e in ev])
        r["third_kernel_median_ms"] = statistics.median([e[3].elapsed_time(e[2]) for e in ev])
    if not cold and form in ("flash", "pf"):
        # GPU time alone: the form's launches replayed back to back from a graph
        if form == "flash":
            fn = lambda: attn.flash(q, k, v, out=out, scale=cfg.scale)
        else:
            def fn():
                attn.stats(q, k, ml=ml, scale=cfg.scale)
                attn.pv(q, k, v, ml, out=out, scale=cfg.scale)
        r["graph_ms"] = _time_graph(fn)
    return r


def config_record(cfg, form: str, steps: int, cold: bool) -> dict:
    """TFLOP/s, % of the MFMA peak and the roofline fraction t_roof / t of one
    config and form (t_roof = max(FLOP / peak, bytes / 8 TB/s))."""
    t = time_steps(cfg, form, steps, 5, cold)
    peak = PEAK_TFLOPS[cfg.dtype]
    by = algorithmic_bytes(cfg, form)
    t_roof = max(cfg.flops / (peak * 1e12), by[form] / (HBM_GBS * 1e9))
    rec = {"config": cfg.name, "variant": form, "dtype": cfg.dtype, "cold": cold,
           "median_us": round(t["median_ms"] * 1e3, 2), "min_us": round(t["min_ms"] * 1e3, 2),
           "tflops": round(cfg.flops / (t["median_ms"] * 1e-3) / 1e12, 2),
           "pct_peak": round(100 * cfg.flops / (t["median_ms"] * 1e-3) / 1e12 / peak, 2),
           "algorithmic_bytes": by[form], "t_roof_us": round(t_roof * 1e6, 3),
           "roofline_frac": round(t_roof / (t["median_ms"] * 1e-3), 4)}
    if "graph_ms" in t:
        tg = t["graph_ms"] * 1e-3
        rec["graph_us"] = round(tg * 1e6, 2)
        rec["graph_tflops"] = round(cfg.flops / tg / 1e12, 2)
        rec["graph_roofline_frac"] = round(t_roof / tg, 4)
    if form in ("pf", "pf_bnhd"):
        ts = t["first_kernel_median_ms"] * 1e-3
        rec["stats_pass_us"] = round(ts * 1e6, 2)
        rec["stats_pass_GBps"] = round(by["stats"] / ts / 1e9, 1)
    if form == "pf_scores":
        for kname, key in (("scores", "first"), ("scores_stats", "second"), ("scores_pv", "third")):
            tk = t[f"{key}_kernel_median_ms"] * 1e-3
            rec[f"{kname}_us"] = round(tk * 1e6, 2)
            rec[f"{kname}_GBps"] = round(by[kname] / tk / 1e9, 1)
    return rec


# The UNet's other specialised kernels at SD 1.x 512x512 (batch 2) sizes, plus
# the 1024x1024 decoder stress (groups of 327680 elements, streamed).
GN_SHAPES = [(2, 320, 64 * 64), (2, 640, 64 * 64), (2, 960, 64 * 64), (2, 1280, 32 * 32),
             (2, 1280, 16 * 16), (2, 2560, 8 * 8), (2, 640, 128 * 128), (8, 320, 64 * 64)]
GEGLU_SHAPES = [(8192, 1280), (2048, 2560), (512, 5120), (128, 5120), (32768, 1280)]


def _time_calls(fn, steps: int, warmup: int = 5):
    """Median and min (ms) of `steps` calls, events around each call."""
    import statistics
    import torch
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for _ in range(warmup):
        fn()
    for e in ev:
        e[0].record(stream)
        fn()
        e[1].record(stream)
    torch.cuda.synchronize()
    t = [e[0].elapsed_time(e[1]) for e in ev]
    return statistics.median(t), min(t)


def _time_graph(fn, calls: int = 20, reps: int = 7):
    """Per-call GPU time (ms) of `calls` back-to-back calls captured in one
    HIP graph (no host work between kernels), median over `reps` replays."""
    import statistics
    import torch
    fn()  # warm-up outside the capture (workspaces, first-use setup)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) / calls)
    return statistics.median(t)


def unet_op_records(steps: int, dtype: str = "f16"):
    """HBM throughput of attn_group_norm and attn_geglu: algorithmic bytes
    (each input read once, each output written once) over the per-call time
    of calls replayed back to back from a HIP graph (these kernels take a few
    µs, less than the host needs to issue a call); the roofline fraction is
    (bytes / 8 TB/s) / time.  median_us / min_us: events around single calls."""
    import torch
    import attention_attn_stats_amd as attn
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    es = {"f16": 2, "bf16": 2, "f32": 4}[dtype]
    g = torch.Generator(device="cuda").manual_seed(0)
    recs = []
    for N, C, HW in GN_SHAPES:
        x = torch.randn((N, C, HW), device="cuda", dtype=torch.float32, generator=g).to(tdt)
        gamma = torch.ones(C, device="cuda", dtype=tdt)
        beta = torch.zeros(C, device="cuda", dtype=tdt)
        y = torch.empty_like(x)
        by = 2 * x.numel() * es + 2 * C * es
        for path in ("auto", "split", "fused", "coop"):
            # 'split' / 'fused' / 'coop' force one form (ATTN_GN_PATH) for comparison
            if path != "auto":
                os.environ["ATTN_GN_PATH"] = path
            fn = (lambda: attn.group_norm(x, 32, gamma, beta, eps=1e-5, out=y))
            med, mn = _time_calls(fn, steps)
            gt = _time_graph(fn)
            os.environ.pop("ATTN_GN_PATH", None)
            recs.append({"op": "group_norm", "shape": [N, C, HW], "groups": 32, "path": path, "dtype": dtype,
                         "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2),
                         "graph_us": round(gt * 1e3, 2), "algorithmic_bytes": by,
                         "GBps_graph": round(by / (gt * 1e-3) / 1e9, 1),
                         "roofline_frac_graph": round(by / (HBM_GBS * 1e9) / (gt * 1e-3), 4)})
    for rows, F in GEGLU_SHAPES:
        h = torch.randn((rows, 2 * F), device="cuda", dtype=torch.float32, generator=g).to(tdt)
        out = torch.empty((rows, F), device="cuda", dtype=tdt)
        by = 3 * rows * F * es
        fn = (lambda: attn.geglu(h, out=out))
        med, mn = _time_calls(fn, steps)
        gt = _time_graph(fn)
        recs.append({"op": "geglu", "shape": [rows, F], "dtype": dtype,
                     "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2),
                     "graph_us": round(gt * 1e3, 2), "algorithmic_bytes": by,
                     "GBps_graph": round(by / (gt * 1e-3) / 1e9, 1),
                     "roofline_frac_graph": round(by / (HBM_GBS * 1e9) / (gt * 1e-3), 4)})
    return recs


def oracle_single_thread(cfg) -> dict:
    """The float64 oracle on one host thread over the whole config (the small
    configs only: a few seconds each), as a per-config CPU reference."""
    import oracle
    from attention_attn_stats_amd import synth
    q, k, v = (synth.widen(x, cfg.dtype) for x in cfg.inputs())
    t0 = time.perf_counter()
    oracle.attention(q, k, v, cfg.scale, nthreads=1)
    t = time.perf_counter() - t0
    return {"oracle_1thread_s": round(t, 4), "oracle_1thread_tflops": round(cfg.flops / t / 1e12, 6)}


SMALL_FOR_ORACLE = ("tiny", "tiny8", "sd512_cross", "level2_self", "level3_self", "level4_self")


def oracle_threads_whole(cfg) -> dict:
    """The float64 oracle over the whole config on the default thread count
    (what a full-output parity check of the config costs)."""
    import oracle
    from attention_attn_stats_amd import synth
    threads = oracle.default_threads()
    q, k, v = (synth.widen(x, cfg.dtype) for x in cfg.inputs())
    t0 = time.perf_counter()
    oracle.attention(q, k, v, cfg.scale, nthreads=threads)
    return {"oracle_threads": threads, "oracle_threads_s": round(time.perf_counter() - t0, 3)}


def oracle_single_thread_sampled(cfg, rows: int = 256) -> dict:
    """The float64 oracle on one host thread over the first `rows` query rows
    of the first head (against all Nk keys), and the whole config's time
    extrapolated from it by rows (every row costs the same Nk-long work)."""
    import oracle
    from attention_attn_stats_amd import synth
    rows = min(rows, cfg.Nq)
    bh = cfg.B * cfg.H
    q, k, v = (synth.widen(x, cfg.dtype).reshape(bh, -1, cfg.d) for x in cfg.inputs())
    t0 = time.perf_counter()
    oracle.attention(q[:1, :rows], k[:1], v[:1], cfg.scale, nthreads=1)
    t = time.perf_counter() - t0
    t_full = t * bh * cfg.Nq / rows
    return {"oracle_1thread_s": round(t_full, 3), "oracle_1thread_tflops": round(cfg.flops / t_full / 1e12, 6),
            "oracle_1thread_extrapolated_from": f"{rows} query rows of one head ({t:.4f} s)"}


def host_cpu() -> dict:
    """The host CPU as /proc/cpuinfo describes it: the model name, family /
    model / stepping, logical CPUs and physical cores (distinct (package,
    core) pairs), and the logical CPUs this process may run on."""
    info = {"model_name": "unknown"}
    pairs, logical, fields = set(), 0, {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" not in ln:
                    if "core id" in fields:
                        pairs.add((fields.get("physical id", "0"), fields["core id"]))
                    fields = {}
                    continue
                k_, v_ = (x.strip() for x in ln.split(":", 1))
                fields[k_] = v_
                if k_ == "processor":
                    logical += 1
                elif k_ in ("model name", "cpu family", "model", "stepping", "vendor_id") and \
                        k_.replace(" ", "_") not in info or (k_ == "model name" and info["model_name"] == "unknown"):
                    info[k_.replace(" ", "_")] = v_
        if "core id" in fields:
            pairs.add((fields.get("physical id", "0"), fields["core id"]))
    except OSError:
        pass
    info["logical_cpus"] = logical or (os.cpu_count() or 0)
    info["physical_cores"] = len(pairs) or None
    try:
        info["cpus_available_to_process"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        info["cpus_available_to_process"] = os.cpu_count()
    return info


def cpu_baseline(cfg, budget_s: float = 20.0):
    """The float64 oracle timed on a bounded sample of the workload: whole
    heads (all Nq query rows against all Nk keys), as many passes over the
    heads as fill about `budget_s` seconds of wall time."""
    import oracle
    from attention_attn_stats_amd import synth
    threads = oracle.default_threads()
    bh = cfg.B * cfg.H
    q, k, v = (synth.widen(x, cfg.dtype).reshape(bh, -1, cfg.d) for x in cfg.inputs())
    t0 = time.perf_counter()
    oracle.attention(q[:1], k[:1], v[:1], cfg.scale, nthreads=threads)
    per_head = max(time.perf_counter() - t0, 1e-3)
    heads = int(min(60 * bh, max(1, budget_s / per_head)))
    done = 0
    t0 = time.perf_counter()
    while done < heads:
        n = min(bh, heads - done)
        oracle.attention(q[:n], k[:n], v[:n], cfg.scale, nthreads=threads)
        done += n
    t = time.perf_counter() - t0
    flops = 4.0 * done * cfg.Nq * cfg.Nk * cfg.d
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "threads_used": threads, "host": host_cpu(),
            "sample": f"{done} head evaluations ({done / bh:.1f} passes over the {bh} heads of {cfg.name}; "
                      f"each {cfg.Nq} queries x {cfg.Nk} keys x d={cfg.d}, float64, score matrix "
                      f"materialised), {t:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="sd512_self")
    ap.add_argument("--variant", default="auto", choices=["auto", "pf", "flash"])
    ap.add_argument("--forms", default="pf,flash,pf_scores",
                    help="forms timed by --configs-out (pf, flash, pf_scores, pf_bnhd, flash_bnhd)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--configs-out", default=None)
    ap.add_argument("--cold", action="store_true")
    ap.add_argument("--unet-ops-out", default=None,
                    help="also time group_norm and geglu at the UNet's sizes, JSONL there")
    ap.add_argument("--sweep-keys", default=None, metavar="NK,NK,...",
                    help="only time the chosen form of --config at each of these key counts "
                         "(seeded inputs, 50 launches each, one JSON line per count) and exit: "
                         "the fixed cost of a dispatch is the intercept")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (calibrates the "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        n = args.copy_probe // 4
        src = torch.ones(n, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4, "launches": 5}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention path is not sharded across GPUs "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from attention_attn_stats_amd.configs import CONFIGS, Config
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = CONFIGS[args.config]
    if args.sweep_keys:
        for nk in (int(x) for x in args.sweep_keys.split(",")):
            c = Config(f"{cfg.name}_nk{nk}", cfg.index, cfg.B, cfg.H, cfg.Nq, nk, cfg.d, cfg.dtype, cfg.sigma_qk,
                       cfg.sigma_v)
            t = time_steps(c, "flash" if args.variant != "pf" else "pf", 50, 5, False)
            print(json.dumps({"config": cfg.name, "Nk": nk, "form": "flash" if args.variant != "pf" else "pf",
                              "median_us": round(t["median_ms"] * 1e3, 2),
                              "graph_us": round(t.get("graph_ms", float("nan")) * 1e3, 2)}), flush=True)
        return
    r = time_config(cfg, args.variant, args.steps, args.warmup)
    flops = cfg.flops
    tflops = flops / (r["ms_per_step"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    # dominant kernel: the one with the largest share of the step
    kname, kms = max(r["kernel_ms"].items(), key=lambda kv: kv[1])
    if kname == "stats":
        kflops = 2.0 * cfg.B * cfg.H * cfg.Nq * cfg.Nk * cfg.d  # Q K^T only
    else:
        kflops = float(flops)  # flash and pv both do Q K^T and P V (pv recomputes Q K^T)
    achieved = kflops / (kms * 1e-3) / 1e12
    kernel_id = {"flash": "attn_flash", "stats": "attn_stats", "pv": "attn_pv"}[kname]
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": load_traffic(kernel_id, cfg),
            "kernel": kernel_id, "kernel_src": os.path.basename(kernel_source(kernel_id, cfg)),
            "kernel_ms": round(kms, 5)}
    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "Nq": cfg.Nq, "Nk": cfg.Nk, "d": cfg.d,
                   "variant": r["variant"], "parallelism": "single GPU"},
        "pct_fp16_mfma_peak": round(100.0 * tflops / PEAK_TFLOPS["f16"], 2),
        "kernel_ms": {k_: round(v_, 5) for k_, v_ in r["kernel_ms"].items()},
        "roofline": roof,
        # time at the binding roof (MFMA here) over the measured step time
        "t_roof_frac": round(max(flops / (peak * 1e12), algorithmic_bytes(cfg, r["variant"])[r["variant"]]
                                 / (HBM_GBS * 1e9)) / (r["ms_per_step"] * 1e-3), 4),
    }
    if args.configs_out:
        with open(args.configs_out, "w") as f:
            import attention_attn_stats_amd as attn
            tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
            for name, c in CONFIGS.items():
                cpu = {"auto_choice": attn.select(c.B, c.H, c.Nq, c.Nk, c.d, tdt[c.dtype])}
                if not args.no_cpu_baseline:
                    cpu.update(oracle_single_thread(c) if name in SMALL_FOR_ORACLE else oracle_single_thread_sampled(c))
                    cpu.update(oracle_threads_whole(c))
                for var in args.forms.split(","):
                    if var == "pf_scores" and c.dtype == "f32":
                        continue  # the stored-logit path runs on the matrix cores only
                    rec = config_record(c, var, max(20, args.steps // 4), args.cold)
                    rec.update(cpu)
                    f.write(json.dumps(rec) + "\n")
                    log(json.dumps(rec))
    if args.unet_ops_out:
        with open(args.unet_ops_out, "w") as f:
            for dt in ("f16", "bf16"):
                for rec in unet_op_records(max(20, args.steps // 4), dt):
                    f.write(json.dumps(rec) + "\n")
                    log(json.dumps(rec))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
