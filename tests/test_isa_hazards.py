"""Matrix-core result hazards in the gfx950 assembly of the library.

The scanner is pinned on small hand-written snippets (each a case the
hardware rules decide), then run over the device assembly of every source
file, compiled with the library's own flags.  CPU only: hipcc cross-compiles.
"""
import shutil

import pytest

from recurrent_attention_amd import build, hazards

MFMA = "v_mfma_f32_16x16x32_bf16"


def _fn(body: str) -> str:
    return "kern:\n" + "\n".join("\t" + l.strip() if not l.strip().endswith(":") else l.strip()
                                 for l in body.strip().splitlines()) + "\n\ts_endpgm\n"


def _check(body):
    return hazards.check_asm(_fn(body))


def test_registers_parse_ranges_and_singles():
    assert hazards.registers("a[0:3], v7, v[10:11]") == {"a0", "a1", "a2", "a3", "v7", "v10", "v11"}
    assert hazards.registers("s[4:5], 0, vcc") == set()


def test_straight_line_read_too_early_is_flagged():
    vs = _check(f"""
        {MFMA} a[0:3], v[2:5], v[6:9], a[0:3]
        s_nop 3
        v_accvgpr_read_b32 v10, a1
    """)
    assert len(vs) == 1 and vs[0].wait_states == 4 and vs[0].required == 8


def test_padded_read_passes():
    assert _check(f"""
        {MFMA} a[0:3], v[2:5], v[6:9], a[0:3]
        s_nop 6
        v_add_u32_e32 v11, v12, v13
        v_accvgpr_read_b32 v10, a1
    """) == []


def test_unrelated_registers_pass():
    assert _check(f"""
        {MFMA} a[0:3], v[2:5], v[6:9], a[0:3]
        v_accvgpr_read_b32 v10, a4
    """) == []


def test_branch_path_that_skips_the_padding_is_flagged():
    # the fall-through block pads enough, the branch target does not
    vs = _check(f"""
        {MFMA} a[0:3], v[2:5], v[6:9], a[0:3]
        s_cbranch_vccnz .LBB0_2
        s_nop 7
        s_nop 7
        s_branch .LBB0_3
.LBB0_2:
        v_mov_b32_e32 v20, 1.0
.LBB0_3:
        v_accvgpr_read_b32 v10, a3
    """)
    assert len(vs) == 1
    assert vs[0].wait_states == 2 and ".LBB0_2" in vs[0].path


def test_loop_back_edge_is_followed():
    vs = _check(f"""
.LBB0_1:
        v_accvgpr_read_b32 v10, a0
        s_nop 7
        {MFMA} a[0:3], v[2:5], v[6:9], a[0:3]
        s_cbranch_scc1 .LBB0_1
    """)
    assert len(vs) == 1 and vs[0].path == [".LBB0_1"]


def test_accumulation_chain_is_forwarded():
    assert _check(f"""
        {MFMA} v[36:39], v[44:47], v[56:59], v[36:39]
        {MFMA} v[34:37], v[40:43], v[44:47], v[36:39]
        {MFMA} v[34:37], v[60:63], v[56:59], v[34:37]
        s_nop 7
        v_cvt_pk_bf16_f32 v34, v34, v35
    """) == []


def test_result_as_multiplicand_is_flagged():
    vs = _check(f"""
        {MFMA} v[36:39], v[44:47], v[56:59], v[36:39]
        {MFMA} v[60:63], v[36:39], v[56:59], 0
    """)
    assert len(vs) == 1


def test_partial_accumulator_overlap_is_flagged():
    vs = _check(f"""
        {MFMA} v[36:39], v[44:47], v[56:59], v[36:39]
        {MFMA} v[60:63], v[40:43], v[44:47], v[34:37]
    """)
    assert len(vs) == 1


def test_fp32_operation_needs_ten():
    body = """
        v_mfma_f32_16x16x4_f32 a[4:7], v2, v21, a[4:7]
        s_nop 7
        v_accvgpr_read_b32 v71, a7
    """
    vs = _check(body)
    assert len(vs) == 1 and vs[0].required == 10 and vs[0].wait_states == 8


def test_unknown_opcode_is_reported():
    vs = _check("""
        v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
        s_nop 7
        s_nop 7
        s_nop 7
    """)
    assert len(vs) == 1 and "missing" in vs[0].reader


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not __import__("os").path.exists(build.HIPCC),
                    reason="hipcc not installed")
def test_library_assembly_has_no_hazards(tmp_path):
    found = build.check_hazards(str(tmp_path))
    assert not found, "\n".join(f"{n}: {v}" for n, v in found[:20])
