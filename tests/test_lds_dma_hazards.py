"""Wait states around the direct global->LDS loads, checked on the generated
gfx950 assembly (CPU only: hipcc cross-compiles the kernel sources to text).

The loads are written as inline assembly, and the compiler inserts no hazard
wait states around inline assembly. Two GFX9 rules apply to them: a vector
memory instruction may read an SGPR (its scalar base address, M0) only five
wait states after a VALU instruction wrote it, and an LDS-DMA load may read
M0 only one wait state after a SALU write. A load that reads a base address
still being written takes a stale one and can fault. Every LDS-DMA load of
every kernel must keep both rules, whatever schedule the compiler picked.
"""

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from fp8_quantized_linear_amd import build as B

VMEM_SGPR_WAIT = 5  # VALU writes an SGPR -> vector memory instruction reads it
M0_LDS_DMA_WAIT = 1  # SALU writes M0 -> LDS-DMA load reads it


def _sources_with_lds_dma():
    out = []
    for s in B.SOURCES:
        text = open(os.path.join(B.CSRC, s)).read()
        if "lds_load16(" in text or "lds_load4(" in text:
            out.append(s)
    return out


def _sgprs(tok):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    if re.fullmatch(r"s\d+|m0", tok):
        return {tok}
    return set()


def _wait_states(ins):
    parts = ins.split()
    return int(parts[1], 0) + 1 if parts[0] == "s_nop" else 1


def _functions(asm):
    """(name, [instruction text or None for a label]) per kernel."""
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.find(".Lfunc_end", m.start())
        body = []
        for line in asm[m.start():end].splitlines()[1:]:
            line = line.split(";")[0].strip()
            if not line or line.startswith("."):
                continue
            body.append(None if line.endswith(":") else line)
        yield m.group(1), body


def hazards(asm):
    """Violations of the two rules in one assembly listing, and the number of
    LDS-DMA loads seen. The look-back is linear and steps over labels, so a
    write in a block that falls or branches into the load's block is seen as
    long as it is the linear predecessor; the loads checked here are preceded
    by an s_nop inside their own asm statement, which no label can split."""
    bad, loads = [], 0
    for name, body in _functions(asm):
        for i, ins in enumerate(body):
            if ins is None:
                continue
            op, *args = ins.replace(",", " ").split()
            if op.startswith("v_") and args and args[0] == "m0":
                bad.append(f"{name}: VALU writes M0: {ins}")
            if not op.startswith("global_load_lds"):
                continue
            loads += 1
            reads = _sgprs(args[1]) | {"m0"}
            waited, j = 0, i - 1
            while j >= 0 and waited < VMEM_SGPR_WAIT:
                prev = body[j]
                j -= 1
                if prev is None:
                    continue
                pop, *pargs = prev.replace(",", " ").split()
                written = _sgprs(pargs[0]) if pargs else set()
                if pop.startswith("v_") and written & reads:
                    bad.append(f"{name}: {prev} {waited} wait states before {ins}")
                if pop.startswith("s_") and "m0" in written and waited < M0_LDS_DMA_WAIT:
                    bad.append(f"{name}: {prev} {waited} wait states before {ins}")
                waited += _wait_states(prev)
    return bad, loads


def test_rules_flag_a_load_right_after_its_base_is_written():
    # the checker itself: a v_readfirstlane into the load's base, and an M0
    # write with no wait state, are both flagged; five wait states clear them
    k = "_Zk:\n"
    bad, n = hazards(k + "\tv_readfirstlane_b32 s53, v3\n\tglobal_load_lds_dword v70, s[52:53]\n.Lfunc_end0:")
    assert n == 1 and len(bad) == 1
    bad, _ = hazards(k + "\ts_mov_b32 m0, s2\n\tglobal_load_lds_dwordx4 v68, s[42:43]\n.Lfunc_end0:")
    assert len(bad) == 1
    bad, _ = hazards(k + "\tv_readfirstlane_b32 s53, v3\n\ts_mov_b32 m0, s2\n\ts_nop 4\n"
                     "\tglobal_load_lds_dword v70, s[52:53]\n.Lfunc_end0:")
    assert bad == []


def _have_hipcc():
    try:
        B._hipcc()
        return True
    except RuntimeError:
        return False


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not installed")
def test_every_lds_dma_load_keeps_its_wait_states(tmp_path):
    sources = _sources_with_lds_dma()
    assert sources, "no kernel source uses the direct global->LDS loads"

    def compile_asm(src):
        out = tmp_path / (src + ".s")
        cmd = [B._hipcc(), *B.HIPCC_FLAGS, "-I", B.CSRC, "--cuda-device-only", "-S",
               os.path.join(B.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, out.read_text()

    with ThreadPoolExecutor(len(sources)) as ex:
        listings = list(ex.map(compile_asm, sources))
    for src, asm in listings:
        bad, loads = hazards(asm)
        assert loads > 0, f"{src}: no LDS-DMA load in the listing"
        assert not bad, f"{src}: " + "\n".join(bad[:20])
