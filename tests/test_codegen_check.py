"""The build's check of the generated assembly (codegen_check.scan) on small
hand-written listings: a register copy between a join label and the restore
of the execution mask is reported; the same copy after the restore, a store
of the branch's body in an out-of-line block, and mask-free lane moves are
not."""
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
