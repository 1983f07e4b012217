"""CPU checks of the build's ISA checks: the hazard checker must flag a DPP
source written by a VALU instruction fewer than two wait states earlier, and
the spill check must flag a hot kernel whose metadata records spills."""

from bitwise_invariant_gated_amd.build import check_dpp_hazards, check_spills


def test_flags_valu_write_right_before_dpp_read():
    asm = """k:
    v_lshlrev_b32_e32 v5, 16, v4
    v_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
"""
    assert len(check_dpp_hazards(asm)) == 1


def test_flags_write_two_instructions_back_without_nop():
    asm = """k:
    v_and_b32_e32 v5, 0xffff0000, v4
    v_mul_f32_e32 v9, s2, v9
    v_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
"""
    assert len(check_dpp_hazards(asm)) == 1


def test_accepts_nop_or_distance():
    ok1 = """k:
    v_lshlrev_b32_e32 v5, 16, v4
    s_nop 1
    v_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
"""
    ok2 = """k:
    v_lshlrev_b32_e32 v5, 16, v4
    v_mul_f32_e32 v9, s2, v9
    v_mul_f32_e32 v8, s2, v8
    v_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
"""
    ok3 = """k:
    v_lshlrev_b32_e32 v6, 16, v4
    v_fmac_f32_dpp v1, v5, v6 row_newbcast:3 row_mask:0xf bank_mask:0xf
"""
    for a in (ok1, ok2, ok3):
        assert check_dpp_hazards(a) == []


def test_register_ranges_count_as_writes():
    asm = """k:
    global_load_dwordx4 v[4:7], v0, s[0:1]
    v_mov_b64 v[4:5], 0
    v_fmac_f32_dpp v1, v5, v2 row_newbcast:0 row_mask:0xf bank_mask:0xf
"""
    assert len(check_dpp_hazards(asm)) == 1


def test_flags_mul_dpp_too():
    asm = """k:
    v_lshlrev_b32_e32 v5, 16, v4
    v_mul_f32_dpp v1, v5, v2 row_newbcast:0 row_mask:0xf bank_mask:0xf
"""
    assert len(check_dpp_hazards(asm)) == 1


def test_spill_check_names_hot_kernels_only():
    meta = """    .name:           _ZN12_GLOBAL__N_113k_resync_bf16ILi128ELi128EEEvNS_10DecodeArgsE
    .private_segment_fixed_size: 224
    .vgpr_count:     168
    .vgpr_spill_count: 55
    .wavefront_size: 64
    .name:           _ZN12_GLOBAL__N_16k_scanIN3cpr3F32ELi128ELi128EEEvNS_11PrefillArgsE
    .vgpr_count:     168
    .vgpr_spill_count: 25
    .wavefront_size: 64
    .name:           _ZN12_GLOBAL__N_16k_scanIN3cpr4Bf16ELi128ELi128EEEvNS_11PrefillArgsE
    .vgpr_count:     166
    .vgpr_spill_count: 0
    .wavefront_size: 64
"""
    bad = check_spills(meta)
    assert [k for _, k in bad] == [55] and "k_resync_bf16" in bad[0][0]


def test_reads_inline_asm_blocks():
    # several instructions in one inline-asm statement are emitted between
    # ASMSTART / ASMEND markers without indentation; a DPP source written by
    # the statement before, or by the instruction before within the
    # statement, is a hazard either way
    before = """k:
	v_lshlrev_b32_e32 v5, 16, v4
	;;#ASMSTART
v_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
v_fmac_f32_dpp v3, v6, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
	;;#ASMEND
"""
    within = """k:
	;;#ASMSTART
v_fmac_f32_dpp v5, v7, v2 row_newbcast:0 row_mask:0xf bank_mask:0xf
v_fmac_f32_dpp v1, v5, v2 row_newbcast:1 row_mask:0xf bank_mask:0xf
	;;#ASMEND
"""
    clean = """k:
	;;#ASMSTART
v_fmac_f32_dpp v1, v5, v2 row_newbcast:0 row_mask:0xf bank_mask:0xf
v_fmac_f32_dpp v3, v6, v1 row_newbcast:0 row_mask:0xf bank_mask:0xf
v_fmac_f32_dpp v1, v5, v8 row_newbcast:1 row_mask:0xf bank_mask:0xf
	;;#ASMEND
"""
    assert len(check_dpp_hazards(before)) == 1
    assert len(check_dpp_hazards(within)) == 1
    assert check_dpp_hazards(clean) == []
