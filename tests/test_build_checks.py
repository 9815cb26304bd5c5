"""The device-code checks of the build (attention_attn_stats_amd/build.py), on
small hand-written gfx950 assembly: an MFMA result read too early on any path
into a block, and a load into an in-flight MFMA's accumulator input, are
found; code that leaves the compiler's own wait states is accepted."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from attention_attn_stats_amd import build  # noqa: E402


def fn(body: str) -> str:
    return "_Z4testv:\n" + body + "\n.Lfunc_end0:\n"


MFMA16 = "\tv_mfma_f32_16x16x32_f16 v[4:7], v[8:11], v[12:15], v[4:7]\n"
MFMA32 = "\tv_mfma_f32_32x32x16_f16 v[16:31], v[8:11], v[12:15], v[16:31]\n"


def test_straight_line_reads_need_the_wait_states_of_the_shape():
    ok16 = fn(MFMA16 + "\ts_nop 7\n\tv_max_f32_e32 v1, v4, v5\n\ts_endpgm")
    short16 = fn(MFMA16 + "\ts_nop 1\n\tv_max_f32_e32 v1, v4, v5\n\ts_endpgm")
    ok32 = fn(MFMA32 + "\ts_nop 7\n\ts_nop 3\n\tv_max_f32_e32 v1, v16, v17\n\ts_endpgm")
    short32 = fn(MFMA32 + "\ts_nop 7\n\tv_max_f32_e32 v1, v16, v17\n\ts_endpgm")
    assert build.early_mfma_result_reads(ok16) == []
    assert len(build.early_mfma_result_reads(short16)) == 1
    assert build.early_mfma_result_reads(ok32) == []
    assert len(build.early_mfma_result_reads(short32)) == 1
    # an LDS read of the result counts as a read; an unrelated register does not
    assert len(build.early_mfma_result_reads(fn(MFMA16 + "\tds_bpermute_b32 v1, v2, v6\n\ts_endpgm"))) == 1
    assert build.early_mfma_result_reads(fn(MFMA16 + "\tv_max_f32_e32 v1, v40, v41\n\ts_endpgm")) == []


def test_a_branch_that_skips_the_padding_is_found():
    # the fall-through path has 12 instructions before the join, the taken
    # branch one: the read at the join is too early on the taken path only
    filler = "".join(f"\tv_mov_b32_e32 v{50 + i}, 0\n" for i in range(12))
    asm = fn(MFMA16 + "\ts_cbranch_scc1 .LBB0_2\n" + filler + ".LBB0_2:\n\tv_max_f32_e32 v1, v6, v7\n\ts_endpgm")
    bad = build.early_mfma_result_reads(asm)
    assert len(bad) == 1 and "v_max_f32" in bad[0]
    # without the branch the same code is fine
    assert build.early_mfma_result_reads(fn(MFMA16 + filler + "\tv_max_f32_e32 v1, v6, v7\n\ts_endpgm")) == []


def test_an_overwritten_result_is_no_longer_tracked():
    asm = fn(MFMA16 + "\ts_nop 7\n\tv_mov_b32_e32 v4, 0\n\tv_max_f32_e32 v1, v4, v4\n\ts_endpgm")
    assert build.early_mfma_result_reads(asm) == []


def test_loads_into_a_pending_accumulator_input_are_found():
    chain = "\tv_mfma_f32_16x16x32_f16 v[20:23], v[8:11], v[12:15], v[4:7]\n"
    bad = build.loads_into_pending_srcc(fn(chain + "\tds_read_b128 v[4:7], v2\n\ts_endpgm"))
    assert len(bad) == 1
    assert build.loads_into_pending_srcc(fn(chain + "\tds_read_b128 v[40:43], v2\n\ts_endpgm")) == []
    far = "".join(f"\tv_mov_b32_e32 v{50 + i}, 0\n" for i in range(build.SRCC_WINDOW + 1))
    assert build.loads_into_pending_srcc(fn(chain + far + "\tds_read_b128 v[4:7], v2\n\ts_endpgm")) == []
