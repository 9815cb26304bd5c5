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

# A load (LDS or memory) whose destination registers were the accumulator
# input of an MFMA issued shortly before can land before that MFMA has read
# them (the MFMA may wait on an earlier one for that very input); on MI355X
# this corrupted single lanes of a short kernel's scores.  The kernels are
# written so that no such pair occurs (loads before products, accumulators
# kept in place); a build that contains one stops.
SRCC_WINDOW = 24  # instructions after an MFMA in which its accumulator input must not be loaded into
_LOAD_OP = re.compile(r"^\s*((?:ds_read|buffer_load|global_load|flat_load)\S*)\s+(v\[\d+:\d+\]|v\d+)")
_MFMA_ANY = re.compile(r"^\s*(v_mfma_\S+)\s+(v\[\d+:\d+\]|v\d+),\s*(\S+),\s*(\S+),\s*(v\[\d+:\d+\]|v\d+)")


def _vregs(spec: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


def loads_into_pending_srcc(asm_text: str, window: int = SRCC_WINDOW) -> list:
    """(MFMA, load) pairs where the load, within `window` instructions after
    the MFMA in the text (labels ignored: a branch may fall through), writes
    registers the MFMA reads as its accumulator input."""
    bad = []
    recent = []  # (index, line, srcC registers) of MFMAs still in the window
    n = 0
    for line in asm_text.splitlines():
        t = line.strip()
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        n += 1
        recent = [r for r in recent if n - r[0] <= window]
        m = _MFMA_ANY.match(t)
        if m:
            recent.append((n, t, _vregs(m.group(5))))
            continue
        lm = _LOAD_OP.match(t)
        if lm:
            dst = _vregs(lm.group(2))
            for _, mt, srcc in recent:
                if dst & srcc:
                    bad.append(mt + "  ->  " + t)
    return bad


# Wait states an MFMA result needs before any other instruction reads it
# (the compiler's own gfx950 figures: passes + 4, 4 passes for 16x16x32 and 8
# for 32x32x16).  The compiler inserts them in straight-line code, but where a
# branch joins it has been seen to count them along one path only (a 16x16x32
# result read 2 wait states after the MFMA on the other path gave single
# wrong query rows on MI355X).  Every path is checked here.
def _result_wait_states(op: str) -> int:
    return 12 if "32x32" in op else 8


_VREF = re.compile(r"v\[(\d+):(\d+)\]|\bv(\d+)\b")


def _vrefs(text: str) -> set:
    out = set()
    for m in _VREF.finditer(text):
        if m.group(1):
            out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _parse_function(body: str):
    """(mnemonic, operand list, text) per instruction, and label -> index."""
    ins, labels = [], {}
    for raw in body.splitlines():
        t = raw.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":"):
            labels[t[:-1]] = len(ins)
            continue
        if t.startswith("."):
            continue
        parts = t.split(None, 1)
        args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        ins.append((parts[0], args, t))
    return ins, labels


def _writes_reads(op: str, args: list):
    """VGPRs an instruction writes and reads (vector ALU, LDS and memory forms)."""
    if not args:
        return set(), set()
    if op.startswith(("v_cmp", "v_cmpx")) and not op.endswith("_e64"):
        return set(), _vrefs(",".join(args))
    if op.startswith(("v_permlane16_swap", "v_permlane32_swap")):
        both = _vrefs(args[0]) | _vrefs(args[1])
        return both, both
    if op.startswith(("v_readfirstlane", "v_readlane")):
        return set(), _vrefs(",".join(args[1:]))
    if op.startswith(("ds_write", "buffer_store", "global_store", "flat_store")):
        return set(), _vrefs(",".join(args))
    if op.startswith(("v_", "ds_", "buffer_load", "global_load", "flat_load")):
        return _vrefs(args[0]), _vrefs(",".join(args[1:]))
    return set(), set()


def early_mfma_result_reads(asm_text: str) -> list:
    """Reads of an MFMA's result by a non-MFMA instruction fewer than the
    needed wait states after it, on any path (branches followed, s_nop N
    counting N + 1)."""
    bad = []
    for fm in re.finditer(r"^(_Z\S*):", asm_text, re.M):
        end = asm_text.find(".Lfunc_end", fm.end())
        ins, labels = _parse_function(asm_text[fm.end():end if end > 0 else len(asm_text)])
        for i, (op, args, text) in enumerate(ins):
            if not op.startswith("v_mfma") or not args:
                continue
            need = _result_wait_states(op)
            stack, seen = [(i + 1, 0, frozenset(_vrefs(args[0])))], set()
            while stack:
                j, states, live = stack.pop()
                if states >= need or not live or j >= len(ins) or (j, states, live) in seen:
                    continue
                seen.add((j, states, live))
                op2, args2, text2 = ins[j]
                w, r = _writes_reads(op2, args2)
                if r & live and not op2.startswith("v_mfma"):
                    bad.append(f"{text}  ->  {text2}  ({states} wait states)")
                    continue
                live2 = live - w
                states2 = states + (int(args2[0], 0) + 1 if op2 == "s_nop" else 1)
                if op2 == "s_endpgm":
                    continue
                target = labels.get(args2[0]) if args2 else None
                if op2.startswith("s_branch"):
                    stack.append((target if target is not None else len(ins), states2, live2))
                    continue
                if op2.startswith("s_cbranch") and target is not None:
                    stack.append((target, states2, live2))
                stack.append((j + 1, states2, live2))
    return bad


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
        bad = loads_into_pending_srcc(text)
        if bad:
            raise RuntimeError(f"loads into an in-flight MFMA's accumulator input in {src}:\n" + "\n".join(bad[:10]))
        bad = early_mfma_result_reads(text)
        if bad:
            raise RuntimeError(f"MFMA results read too early on some path in {src}:\n" + "\n".join(bad[:10]))
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
