"""The build-time hazard check: planted cases in a synthetic disassembly, and
the built library (MFMA hazards in the kernels with inline-assembly MFMAs, SGPR
hazards in every kernel)."""
import os
import shutil

import pytest

from exact_attention_11_amd import hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "exact_attention_11_amd", "libfa2.so")

# Addresses in the comments, as llvm-objdump prints them; the loop branch goes
# back to the second MFMA.
SYNTHETIC = """0000000000001000 <k>:
\tv_mfma_f32_32x32x16_f16 v[0:15], v[16:19], v[20:23], 0      // 000000001000: 0
\tv_mfma_f32_32x32x16_f16 v[0:15], v[16:19], v[20:23], v[0:15] // 000000001008: 0
\ts_nop 7                                                     // 000000001010: 0
\ts_nop 7                                                     // 000000001014: 0
\tv_add_f32_e32 v30, v31, v32                                 // 000000001018: 0
\tv_mov_b32_e32 v17, v2                                       // 00000000101C: 0
\tv_mfma_f32_32x32x16_f16 v[40:55], v[16:19], v[20:23], 0      // 000000001020: 0
\tv_add_f32_e32 v60, v61, v62                                  // 000000001028: 0
\ts_cbranch_scc1 65527                                        // 00000000102C: 0 <k+0x8>
\ts_endpgm                                                    // 000000001030: 0
"""


def test_planted_hazards_are_found():
    insns = hazards.parse(SYNTHETIC)["k"]
    bad = hazards.check_function(insns)
    # the v_mov reads v2 17 wait states after the accumulating MFMA wrote it,
    # and it writes v17 right before the third MFMA reads it; the in-place
    # accumulation itself is not a hazard
    assert ("result", 0x1008, 0x101C, 17) in bad
    assert ("operand", 0x1020, 0x101C, 0) in bad
    assert len(bad) == 2


def test_result_read_across_loop_back_edge():
    dis = """0000000000002000 <k>:
\tv_add_f32_e32 v1, v2, v3                                    // 000000002000: 0
\tv_add_f32_e32 v60, v40, v3                                  // 000000002004: 0
\tv_mfma_f32_32x32x16_f16 v[40:55], v[16:19], v[20:23], 0      // 000000002008: 0
\ts_cbranch_scc1 65532                                        // 000000002010: 0 <k+0x4>
\ts_endpgm                                                    // 000000002014: 0
"""
    bad = hazards.check_function(hazards.parse(dis)["k"])
    assert ("result", 0x2008, 0x2004, 1) in bad


def test_enough_wait_states_pass():
    dis = "0000000000003000 <k>:\n\tv_mfma_f32_32x32x16_f16 v[0:15], v[16:19], v[20:23], 0 // 000000003000: 0\n"
    dis += "".join(f"\ts_nop 7 // {0x3008 + 4 * i:012X}: 0\n" for i in range(3))
    dis += "\tv_add_f32_e32 v30, v3, v32 // 000000003014: 0\n\ts_endpgm // 000000003018: 0\n"
    assert hazards.check_function(hazards.parse(dis)["k"]) == []


# A v_readfirstlane writes the high half of a scalar base that an LDS copy reads
# one instruction later (the form of code that faulted); a second pair is
# separated by s_nop 4 (5 wait states) and passes; a branch carries the third
# write into the loop head's copy.
SGPR_SYNTHETIC = """0000000000004000 <k>:
\tv_readfirstlane_b32 s4, v22                                 // 000000004000: 0
\tv_and_b32_e32 v17, 4, v17                                   // 000000004004: 0
\tv_readfirstlane_b32 s5, v23                                 // 000000004008: 0
\tglobal_load_lds_dwordx4 v6, s[4:5]                          // 00000000400C: 0
\tv_readfirstlane_b32 s14, v20                                // 000000004014: 0
\tv_readfirstlane_b32 s15, v21                                // 000000004018: 0
\ts_nop 4                                                     // 00000000401C: 0
\tglobal_load_lds_dwordx4 v6, s[14:15]                        // 000000004020: 0
\tglobal_load_lds_dwordx4 v7, s[20:21]                        // 000000004028: 0
\tv_cmp_gt_i32_e64 s[20:21], v1, v2                           // 000000004030: 0
\ts_cbranch_scc1 65533                                        // 000000004038: 0 <k+0x28>
\ts_endpgm                                                    // 00000000403C: 0
"""


def test_planted_sgpr_hazards_are_found():
    bad = hazards.check_sgpr_function(hazards.parse(SGPR_SYNTHETIC)["k"])
    assert ("sgpr", 0x4008, 0x400C, 0) in bad  # s5 read right after its write
    assert ("sgpr", 0x4000, 0x400C, 2) in bad  # s4, two wait states earlier
    assert ("sgpr", 0x4030, 0x4028, 1) in bad  # v_cmp's s[20:21] around the loop (the branch between)
    assert len(bad) == 3  # the pair behind s_nop 4 is not reported


def test_sgpr_writers_and_readers():
    ins = hazards.parse(SGPR_SYNTHETIC)["k"]
    assert ins[0].sdst == {4} and ins[3].ssrc == {4, 5} and ins[9].sdst == {20, 21}
    carry = hazards.parse("0000000000005000 <k>:\n\tv_add_co_u32_e64 v1, s[6:7], v2, v3 // 000000005000: 0\n")["k"]
    assert carry[0].sdst == {6, 7}


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(os.path.join(hazards.LLVM_BIN, "llvm-objdump")),
                    reason="library not built or llvm tools missing")
def test_built_library_has_no_hazards():
    assert hazards.check_library(LIB) == []
