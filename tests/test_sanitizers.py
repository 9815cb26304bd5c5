"""CPU-side hardening: the C oracles and the C ABI's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven over edge cases
(tests/sanitize/): any out-of-bounds access, leak or undefined operation fails
the run.  The C ABI's host code is linked against stand-in launchers
(tests/sanitize/host_stubs.cpp) so that no GPU is needed; only host code is
instrumented."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE = os.path.join(ROOT, "oracle")
CSRC = os.path.join(ROOT, "attention_attn_stats_amd", "csrc")
# sanitizer options for the C compiler, and for the HIP compiler's host pass only
C_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0 and "OK" in r.stdout, f"{exe}: rc {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_oracle_c_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", *C_SAN,
                           "-I", ORACLE, os.path.join(SAN, "oracle_driver.c"), os.path.join(ORACLE, "oracle.c"),
                           os.path.join(ORACLE, "unet_ops.c"), "-o", exe, "-lm", "-lpthread"])
    _run(exe)


def test_c_abi_host_code_under_sanitizers(tmp_path):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "host_driver")
    cmd = [hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fno-omit-frame-pointer", *HOST_SAN,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "attn_api.cpp"), os.path.join(SAN, "host_stubs.cpp"), os.path.join(SAN, "host_driver.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    _run(exe)
