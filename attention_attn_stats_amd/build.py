"""Build libattn.so (HIP, gfx950) in-tree with hipcc.

    python -m attention_attn_stats_amd.build
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["attn_api.cpp", "attn_mfma.hip", "attn_fa40.hip", "attn_f32.hip", "attn_scores.hip", "unet_ops.hip",
           "attn_fill.hip", "attn_short.hip"]
ARCH = os.environ.get("ATTN_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    f"--offload-arch={ARCH}",
    # never emit packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs (the softmax reads them on the VALU)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # no NaN operands are expected (IEEE max would otherwise quiet every input first)
    "-fno-honor-nans",
    "-I", INCLUDE, "-I", CSRC,
]

# Flags of one source only.  The attention kernels take the scheduler's
# iterative ILP strategy: the same instructions, ordered for more latency
# hiding; measured -10 % at 256 queries x d = 160, neutral at 4096 x d = 40,
# bit-identical results.
FILE_FLAGS = {
    "attn_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


_MFMA_OP = re.compile(r"^\s*(v_mfma_\S+)")
# MFMA opcodes whose VGPR-form code (accumulator in ordinary VGPRs, chains
# issued back to back, destination allowed to overlap the accumulator input)
# has been checked on gfx950 hardware.  A build that emits any other MFMA
# opcode stops here instead of shipping unverified code: an older-generation
# 16x16x16 op mixed into such chains produced wrong sums.
VERIFIED_MFMA = {"v_mfma_f32_16x16x32_f16", "v_mfma_f32_16x16x32_bf16",
                 "v_mfma_f32_32x32x16_f16", "v_mfma_f32_32x32x16_bf16"}
# For these the ISA forbids a destination that partially overlaps the
# accumulator input (the assembler rejects it); the compiled code is checked.
NO_PARTIAL_OVERLAP = {"v_mfma_f32_32x32x16_f16", "v_mfma_f32_32x32x16_bf16"}
_MFMA_REGS = re.compile(r"^\s*(v_mfma_\S+)\s+v\[(\d+):(\d+)\],\s*\S+,\s*\S+,\s*v\[(\d+):(\d+)\]")


def unverified_mfma(asm_text: str) -> list:
    """MFMA instructions outside VERIFIED_MFMA in the device assembly."""
    bad = []
    for line in asm_text.splitlines():
        m = _MFMA_OP.match(line)
        if m and m.group(1) not in VERIFIED_MFMA:
            bad.append(line.strip())
        r = _MFMA_REGS.match(line)
        if r and r.group(1) in NO_PARTIAL_OVERLAP:
            d0, d1, c0, c1 = (int(r.group(i)) for i in (2, 3, 4, 5))
            if (d0, d1) != (c0, c1) and not (d1 < c0 or c1 < d0):
                bad.append(line.strip() + "    <- partial dst/srcC overlap")
    return bad


MFMA_SOURCES = ["attn_mfma.hip", "attn_fa40.hip", "attn_scores.hip", "attn_short.hip"]


def verify_device_code(hipcc: str, verbose: bool = False, defines=()) -> None:
    """Compile the matrix-core sources to gfx950 assembly and reject unverified MFMA opcodes."""
    total = 0
    for src in MFMA_SOURCES:
        with tempfile.TemporaryDirectory() as td:
            asm = os.path.join(td, src + ".s")
            cmd = [hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), *[f"-D{d}" for d in defines],
                   "-x", "hip", "--cuda-device-only", "-S",
                   os.path.join(CSRC, src), "-o", asm]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"device assembly generation failed for {src}:\n" + r.stderr)
            text = open(asm).read()
        bad = unverified_mfma(text)
        if bad:
            raise RuntimeError(f"unverified MFMA opcodes in {src}:\n" + "\n".join(bad[:10]))
        total += text.count("v_mfma_")
    if verbose:
        print(f"verified {total} MFMA instructions are all of {sorted(VERIFIED_MFMA)}")


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link libattn.so (or `out`) ; returns its path.
    `defines` are extra -D settings of the kernels' compile-time tuning knobs."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    objdir = os.path.join(HERE, "_build", os.path.basename(out))
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), *[f"-D{d}" for d in defines], *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # the host pass does not know the packed-fp32 target feature; that warning is harmless
        msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln
                        and "not a recognized feature" not in ln)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg)
        objs.append(obj)
    verify_device_code(hipcc, verbose, defines)
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
