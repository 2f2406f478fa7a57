"""The device-assembly check for MFMA results read too early
(block_causal_transformer_amd.hazard_check), on hand-written snippets and on
the assembly of the built kernels."""
import glob
import os

import pytest

from block_causal_transformer_amd import hazard_check as H

HEAD = """k:
\tv_mfma_f32_16x16x32_bf16 v[4:7], v[0:3], v[8:11], v[4:7]
\ts_cbranch_vccnz .LBB0_2
\tv_add_u32_e32 v20, 1, v21
\tv_add_u32_e32 v20, 1, v21
\tv_add_u32_e32 v20, 1, v21
\ts_nop 6
.LBB0_2:
"""
TAIL = """\tv_mul_f32_e32 v4, v12, v4
\ts_endpgm
"""


def test_read_after_skipped_block_is_flagged():
    bad = H.check_text(HEAD + TAIL)
    assert "k" in bad and bad["k"][0][2] == 1, bad


def test_enough_wait_states_on_every_path_pass():
    assert H.check_text(HEAD + "\ts_nop 7\n" + TAIL) == {}


def test_unrelated_registers_and_store_sources():
    text = HEAD.replace("s_nop 6", "s_nop 0") + "\tv_mul_f32_e32 v30, v12, v31\n\tds_write_b128 v40, v[4:7]\n\ts_endpgm\n"
    bad = H.check_text(text)
    assert "k" in bad and "ds_write_b128" in bad["k"][0][1]


def test_mfma_chain_is_not_a_hazard():
    text = """k:
\tv_mfma_f32_16x16x32_bf16 v[4:7], v[0:3], v[8:11], 0
\tv_mfma_f32_16x16x32_bf16 v[4:7], v[12:15], v[16:19], v[4:7]
\ts_nop 7
\tv_mul_f32_e32 v4, v12, v4
\ts_endpgm
"""
    assert H.check_text(text) == {}


def test_built_kernels_pass():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    files = glob.glob(os.path.join(root, "_build", "asm", "*.s"))
    if not files:
        pytest.skip("no device assembly built")
    for f in files:
        assert H.check_file(f) == {}, f


def test_32x32_product_needs_twelve_wait_states():
    text = """k:
\tv_mfma_f32_32x32x16_bf16 v[4:19], v[0:3], v[20:23], 0
\ts_nop 7
\tv_mul_f32_e32 v30, v12, v4
\ts_endpgm
"""
    bad = H.check_text(text)
    assert "k" in bad and bad["k"][0][2] == 8, bad
    assert H.check_text(text.replace("s_nop 7", "s_nop 11")) == {}


def test_valu_write_to_result_in_flight_is_flagged():
    text = """k:
\tv_mfma_f32_16x16x32_bf16 v[4:7], v[0:3], v[8:11], 0
\ts_nop 3
\tv_mov_b32_e32 v5, 0
\ts_nop 7
\tv_mul_f32_e32 v30, v12, v4
\ts_endpgm
"""
    bad = H.check_text(text)
    assert "k" in bad and "v_mov_b32" in bad["k"][0][1] and bad["k"][0][2] == 4, bad
    assert H.check_text(text.replace("s_nop 3", "s_nop 7")) == {}


def test_unknown_mfma_opcode_fails():
    text = """k:
\tv_mfma_f32_4x4x4_16b_f16 v[4:7], v[0:1], v[8:9], 0
\ts_nop 15
\tv_mul_f32_e32 v30, v12, v4
\ts_endpgm
"""
    bad = H.check_text(text)
    assert "k" in bad and "unknown MFMA" in bad["k"][0][1]


def test_code_after_an_early_endpgm_is_checked():
    # a kernel with a returning path: the body runs to the function's end
    # marker, not to its first s_endpgm
    text = """k:
\ts_cbranch_scc1 .LBB0_3
\ts_endpgm
.LBB0_3:
\tv_mfma_f32_16x16x32_bf16 v[4:7], v[0:3], v[8:11], v[4:7]
\tv_mul_f32_e32 v4, v12, v4
\ts_endpgm
.Lfunc_end0:
"""
    bad = H.check_text(text)
    assert "k" in bad and "v_mul_f32" in bad["k"][0][1], bad


def test_branch_out_of_the_function_is_an_error():
    with pytest.raises(ValueError):
        H.check_text("k:\n\tv_mfma_f32_16x16x32_bf16 v[4:7], v[0:3], v[8:11], v[4:7]\n"
                     "\ts_branch .LBB9_1\n\ts_endpgm\n.Lfunc_end0:\n")
