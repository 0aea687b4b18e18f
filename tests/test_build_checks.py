"""The build's check of inline-assembly DPP instructions (CPU only): on
synthetic gfx950 disassembly it flags a lane-permuted source written by a VALU
instruction less than two wait states before, on the straight-line path and
along a loop's back edge, and accepts the same code with an s_nop in between;
on the built objects it finds every branch target it needs."""
import os

import pytest

from selective_state_space_27_amd import build as B


def asm(*insts, base=0x1000):
    """llvm-objdump-like lines, one 4-byte word per instruction."""
    return [f"\t{text:<60}// {base + 4 * i:012X}: 00000000" for i, text in enumerate(insts)]


DPP = "v_fmac_f32_dpp v44, v12, v3 row_newbcast:1 row_mask:0xf bank_mask:0xf bound_ctrl:1"


def test_straight_line_hazard_and_nop():
    assert B.dpp_hazards(asm("v_mov_b32_e32 v12, v3", DPP))[1]
    assert B.dpp_hazards(asm("v_mov_b32_e32 v12, v3", "v_add_f32_e32 v5, v6, v7", DPP))[1]
    assert not B.dpp_hazards(asm("v_mov_b32_e32 v12, v3", "s_nop 1", DPP))[1]
    assert not B.dpp_hazards(asm("v_mov_b32_e32 v12, v3", "v_add_f32_e32 v5, v6, v7", "s_nop 0", DPP))[1]
    assert not B.dpp_hazards(asm("buffer_load_dword v12, v1, s[4:7], 0 offen", "s_waitcnt vmcnt(0)", DPP))[1]
    assert B.dpp_hazards(asm("v_pk_mov_b32 v[11:12], v[2:3], v[2:3] op_sel:[0,1]", DPP))[1]  # register range


def test_back_edge_hazard():
    # loop head at index 1 (0x1004); the back edge at index 3 jumps to it:
    # offset = (0x1004 - (0x100c + 4)) / 4 = -3, printed as 65533.
    ok_entry = ["s_nop 1", DPP, "v_add_f32_e32 v5, v6, v7", "s_cbranch_scc1 65533"]
    assert not B.dpp_hazards(asm(*ok_entry))[1]
    bad = ["s_nop 1", DPP, "v_mov_b32_e32 v12, v7", "s_cbranch_scc1 65533"]
    assert B.dpp_hazards(asm(*bad))[1]


@pytest.mark.skipif(not os.path.exists(os.path.join(B.BUILD, "scan.hip.o")), reason="library not built")
def test_built_objects_clean():
    for src in B.DPP_CHECKED:
        seen, bad = B.dpp_hazards(B._disassemble(os.path.join(B.BUILD, src + ".o")))
        assert seen > 0 and not bad, bad[:3]
