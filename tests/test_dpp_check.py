"""The DPP hazard check of the device assembly (CPU only).

The checker is pinned on hand-written gfx950 assembly whose hazards are known
(the gfx9 rule: a DPP instruction may not read a VGPR written in the two
preceding wait states, nor follow a VALU write of EXEC by fewer than five),
then run on the device code of the library's sources, compiled here.
"""
import os
import subprocess
import tempfile

import pytest

from selective_state_space_mssm_amd import dpp_check

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_mssm_amd", "csrc")

DPP = "v_fmac_f32_dpp v10, v1, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf bound_ctrl:1"


def kernel(*body, extra=""):
    lines = ["k:"] + ["\t" + b if not b.endswith(":") else b for b in body] + ["\ts_endpgm", ".Lfunc_end0:"]
    return "\n".join(lines) + extra


def n_hazards(text):
    return len(dpp_check.check_asm(text))


def test_src0_written_just_before():
    assert n_hazards(kernel("v_and_b32_e32 v1, 0xffff0000, v5", DPP)) == 1


def test_one_wait_state_is_not_enough_two_are():
    assert n_hazards(kernel("v_and_b32_e32 v1, 0xffff0000, v5", "s_nop 0", DPP)) == 1
    assert n_hazards(kernel("v_and_b32_e32 v1, 0xffff0000, v5", "s_nop 1", DPP)) == 0
    assert n_hazards(kernel("v_and_b32_e32 v1, 0xffff0000, v5", "v_mov_b32_e32 v7, 0", "s_waitcnt vmcnt(0)",
                            DPP)) == 0


def test_other_source_and_tied_accumulator():
    assert n_hazards(kernel("v_mul_f32_e32 v2, v3, v4", DPP)) == 1   # src1
    assert n_hazards(kernel("v_mul_f32_e32 v10, v3, v4", DPP)) == 1  # fmac accumulator
    # a plain DPP multiply does not read its destination
    mul = "v_mul_f32_dpp v10, v1, v2 row_newbcast:0 row_mask:0xf bank_mask:0xf bound_ctrl:1"
    assert n_hazards(kernel("v_mul_f32_e32 v10, v3, v4", mul)) == 0


def test_register_ranges_and_loads():
    assert n_hazards(kernel("global_load_dwordx4 v[0:3], v[8:9], off", DPP)) == 1  # v1, v2 in the range
    assert n_hazards(kernel("global_load_dwordx4 v[4:7], v[8:9], off", DPP)) == 0
    assert n_hazards(kernel("v_permlane32_swap_b32_e32 v0, v2", DPP)) == 1      # both operands written


def test_unrelated_writes_and_scalar_destinations():
    assert n_hazards(kernel("v_mul_f32_e32 v11, v1, v2", DPP)) == 0
    assert n_hazards(kernel("v_readfirstlane_b32 s1, v1", DPP)) == 0
    assert n_hazards(kernel("v_cmp_gt_f32_e32 vcc, v1, v2", DPP)) == 0


def test_exec_write():
    assert n_hazards(kernel("v_cmpx_gt_f32_e32 vcc, v5, v6", "s_nop 2", DPP)) == 1
    assert n_hazards(kernel("v_cmpx_gt_f32_e32 vcc, v5, v6", "s_nop 4", DPP)) == 0


def test_across_blocks():
    # fall-through predecessor
    assert n_hazards(kernel("v_mov_b32_e32 v1, 0", ".LBB0_1:", DPP)) == 1
    # branch predecessor with enough wait states on one path only
    text = kernel("s_cbranch_scc1 .LBB0_2", "v_mov_b32_e32 v1, 0", "s_branch .LBB0_3",
                  ".LBB0_2:", "v_mov_b32_e32 v1, 1", "s_nop 1", ".LBB0_3:", DPP)
    assert n_hazards(text) == 1
    text = kernel("s_cbranch_scc1 .LBB0_2", "v_mov_b32_e32 v1, 0", "s_nop 1", "s_branch .LBB0_3",
                  ".LBB0_2:", "v_mov_b32_e32 v1, 1", "s_nop 1", ".LBB0_3:", DPP)
    assert n_hazards(text) == 0
    # a loop back edge
    text = kernel(".LBB0_1:", DPP, "v_add_f32_e32 v2, v2, v3", "s_cbranch_scc1 .LBB0_1")
    assert n_hazards(text) == 1


def test_inline_asm_markers_and_comments_are_ignored():
    text = kernel("v_mov_b32_e32 v1, 0 ; comment", ";;#ASMSTART", "s_nop 1", DPP, ";;#ASMEND")
    assert n_hazards(text) == 0


def test_library_device_code_has_no_dpp_hazards():
    """Compile every device source to gfx950 assembly (as the build does) and check it."""
    import __graft_entry__ as entry

    with tempfile.TemporaryDirectory(prefix="mssm_dpp_") as d:
        procs = []
        for src in ("scan_fwd.hip", "scan_conv_fwd.hip", "scan_bwd.hip", "scan_step.hip"):
            cmd = (["hipcc"] + entry.HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                                   "--cuda-device-only", "-S", os.path.join(CSRC, src),
                                                   "-o", os.path.join(d, src + ".s")])
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        for p in procs:
            _, err = p.communicate()
            if p.returncode != 0:
                pytest.fail(err[-2000:])
        total = 0
        for src in ("scan_fwd.hip", "scan_conv_fwd.hip", "scan_bwd.hip"):
            text = open(os.path.join(d, src + ".s")).read()
            assert dpp_check.check_asm(text) == []
            total += dpp_check.count_dpp(text)
        assert total > 1000  # the kernels do use DPP: the check had something to check
