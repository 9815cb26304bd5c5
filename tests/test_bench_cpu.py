"""The measurement code of bench.py, on the CPU: the one-GPU contract, the
algorithmic work it divides by (checked against the per-config figures of the
workload table, worked out by hand from the shapes: FLOP = 4 B H Nq Nk d; flash
bytes = Q + K + V + O; two-pass bytes = 2Q + 2K + V + O + 2 ml; stats-pass bytes
= Q + K + ml, 2-byte elements and 8-byte (m, l) rows), and the rule that stored
traffic counters are reported only for the kernel source and flags they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from attention_attn_stats_amd.configs import CONFIGS  # noqa: E402

# (scores, FLOP, flash bytes, two-pass bytes, stats-pass bytes)
TABLE = {
    "sd512_self": (268_435_456, 42_949_672_960, 20_971_520, 32_505_856, 11_010_048),
    "sd512_cross": (5_046_272, 807_403_520, 10_682_880, 17_072_896, 5_865_728),
    "level2_self": (16_777_216, 5_368_709_120, 10_485_760, 15_990_784, 5_373_952),
    "level3_self": (1_048_576, 671_088_640, 5_242_880, 7_929_856, 2_654_208),
    "level4_self": (65_536, 41_943_040, 1_310_720, 1_982_464, 663_552),
    "sd1024_self": (4_294_967_296, 687_194_767_360, 83_886_080, 130_023_424, 44_040_192),
}


@pytest.mark.parametrize("name", sorted(TABLE))
def test_algorithmic_work_matches_the_table(name):
    cfg = CONFIGS[name]
    scores, flops, flash_b, pf_b, stats_b = TABLE[name]
    assert cfg.B * cfg.H * cfg.Nq * cfg.Nk == scores
    assert cfg.flops == flops
    by = bench.algorithmic_bytes(cfg, "flash")
    assert by["flash"] == flash_b
    assert by["pf"] == pf_b
    assert by["stats"] == stats_b
    assert by["flash_bnhd"] == flash_b and by["pf_bnhd"] == pf_b  # the strided forms move the same bytes


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    from attention_attn_stats_amd.configs import CONFIGS
    cfg = CONFIGS["sd512_self"]
    src = tmp_path / "kernel.hip"
    src.write_text("int f() {\n  return 1;  // one\n}\n/* block */\n")
    monkeypatch.setattr(bench, "kernel_source", lambda kernel, c: str(src))
    h = bench.kernel_hash(str(src))
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps({"attn_flash@sd512_self": {"kernel_src_sha256_16": h, "bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.load_traffic("attn_flash", cfg) == 123
    # comments and blank space do not count ...
    src.write_text("int f() {\n\n    return 1;  // changed comment\n}\n/* other */\n")
    assert bench.kernel_hash(str(src)) == h and bench.load_traffic("attn_flash", cfg) == 123
    # ... code does
    src.write_text("int f() {\n  return 2;\n}\n")
    assert bench.kernel_hash(str(src)) != h and bench.load_traffic("attn_flash", cfg) is None
    assert bench.load_traffic("attn_flash", CONFIGS["sd1024_self"]) is None
    # ... and so do compile flags given to that file alone
    from attention_attn_stats_amd import build
    h2 = bench.kernel_hash(str(src))
    monkeypatch.setitem(build.FILE_FLAGS, "kernel.hip", ["-mllvm", "-some-option"])
    assert bench.kernel_hash(str(src)) != h2


def test_kernel_source_follows_the_dispatch(monkeypatch):
    from attention_attn_stats_amd.configs import CONFIGS
    monkeypatch.delenv("ATTN_FA40", raising=False)
    monkeypatch.delenv("ATTN_SHORT", raising=False)
    c1 = CONFIGS["sd512_self"]
    assert bench.kernel_source("attn_flash", c1).endswith("attn_fa40.hip")
    assert bench.kernel_source("attn_pv", c1).endswith("attn_fa40.hip")
    assert bench.kernel_source("attn_stats", c1).endswith("attn_mfma.hip")
    assert bench.kernel_source("attn_flash", CONFIGS["level2_self"]).endswith("attn_mfma.hip")  # 1024 keys
    assert bench.kernel_source("attn_flash", CONFIGS["sd1024_self"]).endswith("attn_fa40.hip")  # 16384 keys
    for name in ("sd512_cross", "level3_self", "level4_self"):  # 77, 256, 64 keys
        assert bench.kernel_source("attn_flash", CONFIGS[name]).endswith("attn_short.hip")
        assert bench.kernel_source("attn_pv", CONFIGS[name]).endswith("attn_mfma.hip")
    assert bench.kernel_source("attn_flash", CONFIGS["tiny"]).endswith("attn_mfma.hip")  # f32: not the MFMA kernels
    monkeypatch.setenv("ATTN_FA40", "1")
    assert bench.kernel_source("attn_flash", CONFIGS["sd1024_self"]).endswith("attn_fa40.hip")
    assert bench.kernel_source("attn_flash", CONFIGS["sd512_cross"]).endswith("attn_short.hip")
    monkeypatch.setenv("ATTN_SHORT", "0")
    assert bench.kernel_source("attn_flash", CONFIGS["sd512_cross"]).endswith("attn_fa40.hip")
    monkeypatch.setenv("ATTN_FA40", "0")
    assert bench.kernel_source("attn_flash", c1).endswith("attn_mfma.hip")
    assert bench.kernel_source("attn_flash", CONFIGS["level4_self"]).endswith("attn_mfma.hip")
