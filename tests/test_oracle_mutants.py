"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/oracle.c, plants one plausible slip (on the CPU, in a
temporary directory), builds it and runs tests/test_oracle_pins.py against the
broken build in a subprocess; the pin suite has to fail.  The unmodified
source must pass the same way.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "dropped_scale": ("s[(size_t)i * nk + j] = scale * acc;", "s[(size_t)i * nk + j] = acc;"),
    "exponent_sign": ("sum += exp(row[j] - mx);", "sum += exp(mx - row[j]);"),
    "p_not_normalised": ("exp(row[j] - mx) / sum;", "exp(row[j] - mx);"),
    "v_transposed": ("acc += p[(size_t)i * nk + j] * v[(size_t)j * d + c];",
                     "acc += p[(size_t)i * nk + j] * v[(size_t)c * nk + j];"),
    "k_transposed": ("acc += q[(size_t)i * d + c] * k[(size_t)j * d + c];",
                     "acc += q[(size_t)i * d + c] * k[(size_t)c * nk + j];"),
    "max_skips_last_key": ("for (int j = 1; j < nk; ++j)\n      if (row[j] > mx) mx = row[j];",
                           "for (int j = 1; j < nk - 1; ++j)\n      if (row[j] > mx) mx = row[j];"),
    "merge_factor_inverted": ("l = (l > 0.0 ? l * exp(m - mm) : 0.0) + bl * exp(bm - mm);",
                              "l = (l > 0.0 ? l * exp(mm - m) : 0.0) + bl * exp(bm - mm);"),
    "l_reported_inverse": ("l[i] = sum;", "l[i] = 1.0 / sum;"),
}


def _run_pins(tmp_path, source: str) -> int:
    c = tmp_path / "oracle.c"
    c.write_text(source)
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                           "-I", os.path.join(ROOT, "oracle"), str(c), "-o", str(so), "-lm", "-lpthread"])
    env = dict(os.environ, ATTN_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
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
