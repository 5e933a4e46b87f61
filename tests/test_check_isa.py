"""The build-time machine-code check on MFMA result overlaps (host only)."""
from gated_delta_rule_prologue_amd import check_isa

HEAD = "_ZN5prism4testEv:\n"


def test_flags_mixed_shape_pair_two_registers_apart():
    asm = HEAD + """
\tv_mfma_f32_16x16x32_bf16 v[136:139], v[80:83], v[20:23], v[150:153]
\tv_mfma_f32_16x16x16_bf16 v[138:141], v[134:135], v[32:33], v[136:139]
"""
    assert len(check_isa.scan(asm)) == 1


def test_flags_the_reverse_order_too():
    asm = HEAD + """
\tv_mfma_f32_16x16x16_bf16 v[136:139], v[134:135], v[32:33], v[150:153]
\tv_mfma_f32_16x16x32_bf16 v[138:141], v[80:83], v[20:23], v[136:139]
"""
    assert len(check_isa.scan(asm)) == 1


def test_accepts_same_shape_offset_pairs():
    asm = HEAD + """
\tv_mfma_f32_16x16x32_bf16 v[52:55], v[74:77], v[64:67], v[0:3]
\tv_mfma_f32_16x16x32_bf16 v[50:53], v[74:77], v[64:67], v[52:55]
"""
    assert check_isa.scan(asm) == []


def test_accepts_in_place_and_disjoint_results():
    asm = HEAD + """
\tv_mfma_f32_16x16x32_bf16 v[136:139], v[80:83], v[20:23], v[136:139]
\tv_mfma_f32_16x16x16_bf16 v[136:139], v[134:135], v[32:33], v[136:139]
\tv_mfma_f32_16x16x16_bf16 v[140:143], v[134:135], v[32:33], v[140:143]
\tv_mfma_f32_16x16x16_bf16 v[40:43], v[134:135], v[32:33], v[40:43]
\tv_mfma_f32_16x16x32_bf16 v[42:45], v[80:83], v[20:23], v[42:45]
"""
    assert check_isa.scan(asm) == []


def test_window_and_function_boundaries():
    far = "".join("\tv_add_f32_e32 v1, v2, v3\n" for _ in range(check_isa.WINDOW + 1))
    asm = HEAD + "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[8:11], v[8:11], v[0:3]\n" + far + \
        "\tv_mfma_f32_16x16x16_bf16 v[2:5], v[8:9], v[8:9], v[0:3]\n"
    assert check_isa.scan(asm) == []
    asm2 = HEAD + "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[8:11], v[8:11], v[0:3]\n" + \
        "_ZN5prism5otherEv:\n\tv_mfma_f32_16x16x16_bf16 v[2:5], v[8:9], v[8:9], v[0:3]\n"
    assert check_isa.scan(asm2) == []


def test_flags_dpp_source_written_just_before():
    asm = HEAD + """
\tv_lshlrev_b32_e32 v75, 16, v66
\tv_fmac_f32_dpp v58, v75, -v102 row_newbcast:1 row_mask:0xf bank_mask:0xf
"""
    assert len(check_isa.scan_dpp(asm)) == 1


def test_flags_dpp_source_one_wait_state_short():
    asm = HEAD + """
\tv_lshlrev_b32_e32 v75, 16, v66
\tv_mov_b32_e32 v1, v2
\tv_fmac_f32_dpp v58, v75, -v102 row_newbcast:2 row_mask:0xf bank_mask:0xf
"""
    assert len(check_isa.scan_dpp(asm)) == 1


def test_accepts_dpp_after_nop_or_two_other_instructions():
    asm = HEAD + """
\tv_lshlrev_b32_e32 v75, 16, v66
\t;;#ASMSTART
\ts_nop 1
\tv_fmac_f32_dpp v58, v75, -v102 row_newbcast:1 row_mask:0xf bank_mask:0xf
\t;;#ASMEND
\tv_lshlrev_b32_e32 v76, 16, v67
\tv_mov_b32_e32 v1, v2
\tv_and_b32_e32 v3, 1, v4
\tv_fmac_f32_dpp v59, v76, -v102 row_newbcast:1 row_mask:0xf bank_mask:0xf
\tv_add_f32_dpp v5, v9, v9 row_shr:1 row_mask:0xf bank_mask:0xf
"""
    assert check_isa.scan_dpp(asm) == []
