"""The build's check of the generated assembly (codegen_check.scan) on small
hand-written listings: a register copy between a join label and the restore
of the execution mask is reported; the same copy after the restore, a store
of the branch's body in an out-of-line block, mask-free lane moves, and code
after a guard branch that left the mask as it was are not."""
from causal_gqa_attention_bwd_amd.codegen_check import scan

HEAD = """_Z6kernelv:
	s_and_saveexec_b64 s[6:7], vcc
	s_cbranch_execz .LBB0_2
; %bb.1:
	global_load_dword a76, v[4:5], off
"""


def test_copy_before_the_mask_restore_is_reported():
    asm = HEAD + """.LBB0_2:
	v_accvgpr_write_b32 a78, v15
	s_or_b64 exec, exec, s[6:7]
	s_endpgm
"""
    hits = scan(asm)
    assert len(hits) == 1
    name, _, ins = hits[0]
    assert name == "_Z6kernelv" and ins == ["v_accvgpr_write_b32 a78, v15"]


def test_copy_after_the_mask_restore_is_fine():
    asm = HEAD + """.LBB0_2:
	s_or_b64 exec, exec, s[6:7]
	v_accvgpr_write_b32 a78, v15
	s_endpgm
"""
    assert scan(asm) == []


def test_out_of_line_body_and_lane_moves_are_fine():
    # a then-block reached by s_cbranch_execnz holds the body's own stores;
    # v_writelane ignores the mask
    asm = """_Z6kernelv:
	s_and_saveexec_b64 s[2:3], vcc
	s_cbranch_execnz .LBB0_7
.LBB0_3:
	v_writelane_b32 v255, s8, 52
	s_or_b64 exec, exec, s[2:3]
	s_endpgm
.LBB0_7:
	v_accvgpr_read_b32 v0, a86
	global_store_dword v[0:1], v50, off
	s_or_b64 exec, exec, s[2:3]
	s_branch .LBB0_3
"""
    assert scan(asm) == []


def test_guard_branch_that_keeps_the_mask_marks_no_join():
    # s_cbranch_execz over a zero-fill with no mask write before it: the
    # target runs with the mask of the code before, whatever comes later
    asm = """_Z6kernelv:
	s_cmp_lt_i32 s4, 1
	s_cbranch_scc1 .LBB0_9
.LBB0_1:
	s_load_dwordx2 s[6:7], s[0:1], 0x30
	s_cbranch_execz .LBB0_3
; %bb.2:
	v_mov_b32_e32 v2, 0
.LBB0_3:
	v_mul_f32_e32 v18, s29, v18
	v_cmp_lt_u32_e64 s[4:5], v34, v35
	s_and_saveexec_b64 s[2:3], s[4:5]
; %bb.5:
	v_mov_b32_e32 v56, v19
; %bb.6:
	s_or_b64 exec, exec, s[2:3]
	s_endpgm
.LBB0_9:
	s_endpgm
"""
    assert scan(asm) == []


def test_mask_write_earlier_in_the_run_still_marks_the_join():
    # the narrowing sits before a uniform branch of the same straight run
    asm = """_Z6kernelv:
	s_and_saveexec_b64 s[6:7], vcc
	s_cbranch_vccnz .LBB0_9
	s_cbranch_execz .LBB0_2
; %bb.1:
	global_load_dword a76, v[4:5], off
.LBB0_2:
	v_accvgpr_write_b32 a78, v15
	s_or_b64 exec, exec, s[6:7]
	s_endpgm
.LBB0_9:
	s_endpgm
"""
    assert len(scan(asm)) == 1
