"""Wait states before the direct global->LDS loads, checked on the generated
gfx950 assembly (CPU only: hipcc cross-compiles the kernel sources to text).

The loads are inline assembly, around which the compiler inserts no hazard
wait states. Two GFX9 rules apply: a vector memory instruction may read an
SGPR (its scalar base address, M0) only five wait states after a VALU
instruction wrote it, and an LDS-DMA load may read M0 only one wait state
after a SALU write. A load that reads a base address still being written
takes a stale one and can fault. build() runs the same check and refuses to
link a library that breaks either rule; here the checker itself is tested on
small listings, then run on every kernel source that issues such loads.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import pytest

from fp8_quantized_linear_amd import build as B
from fp8_quantized_linear_amd.lds_dma_check import device_asm, hazards, sources_with_lds_dma


def _listing(*lines):
    return "_Zk:\n" + "".join(f"{l}\n" if l.endswith(":") else f"\t{l}\n" for l in lines) + ".Lfunc_end0:"


def test_a_load_right_after_its_base_or_m0_is_written_is_flagged():
    bad, n = hazards(_listing("v_readfirstlane_b32 s53, v3", "global_load_lds_dword v70, s[52:53]"))
    assert n == 1 and len(bad) == 1
    bad, _ = hazards(_listing("s_mov_b32 m0, s2", "global_load_lds_dwordx4 v68, s[42:43]"))
    assert len(bad) == 1
    bad, _ = hazards(_listing("v_readfirstlane_b32 m0, v1", "s_nop 3", "global_load_lds_dword v1, s[2:3]"))
    assert len(bad) == 2  # a VALU write of M0, four wait states before the load


def test_enough_wait_states_clear_both_rules():
    assert hazards(_listing("v_readfirstlane_b32 s53, v3", "s_mov_b32 m0, s2", "s_nop 3",
                            "global_load_lds_dword v70, s[52:53]"))[0] == []
    assert hazards(_listing("s_mov_b32 m0, s2", "s_nop 0", "global_load_lds_dword v70, s[52:53]"))[0] == []
    # a VALU that only reads the SGPR is no hazard
    assert hazards(_listing("v_add_u32_e32 v1, s52, v2", "s_nop 0", "global_load_lds_dword v70, s[52:53]"))[0] == []


def test_carry_outputs_count_as_sgpr_writes():
    bad, _ = hazards(_listing("v_add_co_u32_e64 v1, s[52:53], v2, v3", "s_nop 1",
                              "global_load_lds_dword v70, s[52:53]"))
    assert len(bad) == 1
    bad, _ = hazards(_listing("v_cmp_lt_i64_e32 vcc, v[2:3], v[4:5]", "s_nop 0",
                              "global_load_lds_dword v70, vcc"))
    assert len(bad) == 1


def test_the_look_back_follows_branches_into_the_load_block():
    # the linear predecessor has waited long enough, the branch source has not
    listing = _listing("v_readfirstlane_b32 s53, v3", "s_cbranch_scc1 .LBB0_2", "s_nop 7", "s_nop 7",
                       ".LBB0_2:", "s_nop 0", "global_load_lds_dword v70, s[52:53]")
    bad, _ = hazards(listing)
    assert len(bad) == 1 and "v_readfirstlane_b32 s53" in bad[0]
    # after an unconditional branch the label is not reached by falling through
    listing = _listing("v_readfirstlane_b32 s53, v3", "s_branch .LBB0_3", ".LBB0_2:", "s_nop 0",
                       "global_load_lds_dword v70, s[52:53]", ".LBB0_3:", "s_endpgm")
    assert hazards(listing)[0] == []
    # a loop back-edge: the write at the loop's end reaches the load at its head
    listing = _listing("s_nop 7", ".LBB0_1:", "s_nop 0", "global_load_lds_dword v70, s[52:53]", "s_nop 7",
                       "v_readfirstlane_b32 s52, v3", "s_cbranch_scc1 .LBB0_1")
    assert len(hazards(listing)[0]) == 1


def _have_hipcc():
    try:
        B._hipcc()
        return True
    except RuntimeError:
        return False


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not installed")
def test_every_lds_dma_load_keeps_its_wait_states(tmp_path):
    sources = sources_with_lds_dma(B.CSRC, B.SOURCES)
    assert sources, "no kernel source uses the direct global->LDS loads"

    def compile_asm(src):
        return src, device_asm(B._hipcc(), B.HIPCC_FLAGS, B.CSRC, src, str(tmp_path / (src + ".s")))

    with ThreadPoolExecutor(len(sources)) as ex:
        listings = list(ex.map(compile_asm, sources))
    for src, asm in listings:
        bad, loads = hazards(asm)
        assert loads > 0, f"{src}: no LDS-DMA load in the listing"
        assert not bad, f"{src}: " + "\n".join(bad[:20])
