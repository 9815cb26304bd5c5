"""Planted mistakes in the group-normalisation / gated-GELU oracle must be
caught by its pins.

Each case copies oracle/unet_ops.c, plants one plausible slip (on the CPU, in
a temporary directory), builds it and runs tests/test_oracle_ops_pins.py
against the broken build in a subprocess; the pin suite has to fail.  The
unmodified source must pass the same way.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "unet_ops.c")

MUTANTS = {
    "unbiased_variance": ("const double var = sq / (double)len;", "const double var = sq / (double)(len - 1);"),
    "eps_outside_sqrt": ("1.0 / sqrt(var + eps);", "1.0 / (sqrt(var) + eps);"),
    "deviation_without_mean": ("const double dev = x[base + e] - mean;", "const double dev = x[base + e];"),
    "gamma_per_group": ("gamma ? gamma[cc] : 1.0;", "gamma ? gamma[g] : 1.0;"),
    "beta_dropped": ("y[i] = (x[i] - mean) * rstd * ga + be;", "y[i] = (x[i] - mean) * rstd * ga;"),
    "groups_strided": ("const size_t i = base + (size_t)ch * hw + p;",
                       "const size_t i = ((size_t)s * c + (size_t)ch * groups + g) * hw + p;"),
    "gelu_no_sqrt2": ("erfc(-x / sqrt(2.0))", "erfc(-x)"),
    "gelu_no_half": ("return 0.5 * x * erfc", "return x * erfc"),
    "gelu_sign": ("erfc(-x / sqrt(2.0))", "erfc(x / sqrt(2.0))"),
    "geglu_halves_swapped": ("row[j] * oracle_gelu1(row[f + j])", "row[f + j] * oracle_gelu1(row[j])"),
    "geglu_gate_reversed": ("row[j] * oracle_gelu1(row[f + j])", "row[j] * oracle_gelu1(row[2 * f - 1 - j])"),
}


def _run_pins(tmp_path, source: str) -> int:
    c = tmp_path / "unet_ops.c"
    c.write_text(source)
    so = tmp_path / "liboracle_ops_mut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                           "-I", os.path.join(ROOT, "oracle"), str(c), "-o", str(so), "-lm"])
    env = dict(os.environ, ATTN_ORACLE_OPS_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_ops_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode


def test_unmodified_source_passes(tmp_path):
    assert _run_pins(tmp_path, open(SRC).read()) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not found exactly once"
    assert _run_pins(tmp_path, src.replace(before, after)) != 0, f"pins did not catch {name}"
