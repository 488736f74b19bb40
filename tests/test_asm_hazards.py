"""The operand-hazard check of the inline-asm MFMAs: the checker itself on hand-made
sequences, and the compiled gfx950 code of the step-2 kernels (no GPU needed)."""
import os

from flashattention_backward_amd import asm_check, build

MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[32:35], v[40:43], a[0:15]"


def test_vector_write_right_before_is_a_hazard():
    asm = "v_cvt_pk_bf16_f32 v35, v1, v2\n" + MFMA
    assert len(asm_check.mfma_operand_hazards(asm)) == 1


def test_two_wait_states_clear_it():
    assert asm_check.mfma_operand_hazards("v_cvt_pk_bf16_f32 v35, v1, v2\ns_nop 1\n" + MFMA) == []
    assert asm_check.mfma_operand_hazards(
        "v_cvt_pk_bf16_f32 v35, v1, v2\nv_add_u32_e32 v7, 1, v7\nds_read_b128 v[8:11], v3\n" + MFMA) == []


def test_one_wait_state_is_not_enough():
    asm = "v_cvt_pk_bf16_f32 v41, v1, v2\ns_nop 0\n" + MFMA
    assert len(asm_check.mfma_operand_hazards(asm)) == 1
    asm = "v_cvt_pk_bf16_f32 v41, v1, v2\nv_add_u32_e32 v7, 1, v7\n" + MFMA
    assert len(asm_check.mfma_operand_hazards(asm)) == 1


def test_accumulator_moves_and_srcc_count():
    assert len(asm_check.mfma_operand_hazards("v_accvgpr_read_b32 v42, a7\n" + MFMA)) == 1
    assert len(asm_check.mfma_operand_hazards("v_accvgpr_write_b32 a3, v9\n" + MFMA)) == 1


def test_unrelated_writes_are_not_hazards():
    asm = "v_cmp_gt_i32_e32 vcc, 18, v35\nv_mov_b32_e32 v44, v1\n" + MFMA
    assert asm_check.mfma_operand_hazards(asm) == []


def test_compiled_step2_kernels_have_no_mfma_operand_hazard():
    path = build.device_asm_path("bwd16.hip")
    if not os.path.exists(path):
        os.makedirs(build.BUILD, exist_ok=True)
        build._compile("bwd16.hip")  # raises on a hazard as well
    asm = open(path).read()
    assert asm_check.count_mfma(asm) > 100
    assert asm_check.mfma_operand_hazards(asm) == []
