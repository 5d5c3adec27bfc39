"""The build check for MFMA operand hazards that inline asm hides from the compiler.

The attend kernels issue MFMAs from inline asm without the two wait states a
VALU-written operand would need; isa_check scans the compiled code for any
such write.  These tests pin the checker on small hand-written sequences (it
must flag a VALU write of an operand one or no wait state before an MFMA, in
the same block or across a branch, and must accept loads and padded writes),
then run it on the library source.
"""
import os
import shutil

import pytest

from mla_latent_cache_absorbed_amd import isa_check as ic
from mla_latent_cache_absorbed_amd import build as b

MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]"


def _k(*body):
    return "_Zk:\n" + "\n".join("\t" + x for x in body) + "\n\ts_endpgm\n"


def test_flags_valu_write_just_before():
    assert len(ic.check_asm(_k("v_mov_b32 v1, v9", MFMA))) == 1
    assert len(ic.check_asm(_k("v_add_f32_e32 v6, v7, v8", MFMA))) == 1   # source B
    assert len(ic.check_asm(_k("v_accvgpr_write_b32 a3, v9", MFMA))) == 1  # accumulator


def test_flags_write_one_wait_state_away():
    assert len(ic.check_asm(_k("v_mov_b32 v1, v9", "s_nop 0", MFMA))) == 1
    assert len(ic.check_asm(_k("v_mov_b32 v1, v9", "s_mov_b32 s0, 1", MFMA))) == 1


def test_accepts_two_wait_states_and_loads():
    assert ic.check_asm(_k("v_mov_b32 v1, v9", "s_nop 1", MFMA)) == []
    assert ic.check_asm(_k("v_mov_b32 v1, v9", "s_nop 0", "s_nop 0", MFMA)) == []
    assert ic.check_asm(_k("v_mov_b32 v20, v9", MFMA)) == []  # unrelated register
    assert ic.check_asm(_k("ds_read_b128 v[0:3], v9", "s_waitcnt lgkmcnt(0)", MFMA)) == []
    assert ic.check_asm(_k("v_cmp_lt_f32_e32 vcc, v1, v2", MFMA)) == []  # writes no vector register


def test_follows_branches_into_the_block():
    asm = ("_Zk:\n\tv_mov_b32 v2, 0\n\ts_branch .LBB0_2\n.LBB0_1:\n\ts_nop 7\n"
           ".LBB0_2:\n\t" + MFMA + "\n\ts_cbranch_scc1 .LBB0_1\n\ts_endpgm\n")
    probs = ic.check_asm(asm)
    assert len(probs) == 1 and "v_mov_b32 v2, 0" in probs[0]
    # the same with the write two wait states away on every path
    ok = asm.replace("\ts_branch .LBB0_2\n", "\ts_nop 0\n\ts_branch .LBB0_2\n")
    assert ic.check_asm(ok) == []


@pytest.mark.skipif(not shutil.which(b.HIPCC) and not os.path.exists(b.HIPCC), reason="hipcc not available")
def test_library_has_no_mfma_operand_hazards():
    assert ic.check_source(b.SRC, b.HIPCC, b.FLAGS) == []
