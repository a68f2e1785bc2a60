"""Build-time check of the wait states before the direct global->LDS loads.

The loads (global_load_lds_dword / _dwordx4) are written as inline assembly,
and the compiler inserts no hazard wait states around inline assembly. Two
GFX9 rules apply to them:
  * a vector memory instruction may read an SGPR (its scalar base address,
    and M0, which carries the LDS address) only five wait states after a VALU
    instruction wrote it;
  * an LDS-DMA load may read M0 only one wait state after a SALU write.
Each asm statement opens with s_nop 0, which keeps the second rule in every
schedule. The first depends on where the compiler put the VALU instructions
that produce the base (v_readfirstlane, 64-bit compares and selects), so it
is checked here on the generated assembly of every kernel source that uses
the loads; build() refuses to link a library with a violation. A load that
reads a base address still being written takes a stale one and can fault.
"""

import os
import re
import subprocess

VMEM_SGPR_WAIT = 5   # VALU writes an SGPR -> vector memory instruction reads it
M0_LDS_DMA_WAIT = 1  # SALU writes M0 -> LDS-DMA load reads it
VCC = ("s106", "s107")  # VCC is SGPR 106-107 on GFX9

# VALU instructions with a scalar carry or condition output: in the VOP3 form
# (_e64) it is the second operand, in the VOP2 form it is VCC
_CARRY_OPS = ("v_add_co_u32", "v_sub_co_u32", "v_subrev_co_u32", "v_addc_co_u32",
              "v_subb_co_u32", "v_subbrev_co_u32", "v_div_scale_f32", "v_div_scale_f64",
              "v_mad_u64_u32", "v_mad_i64_i32")
_UNCONDITIONAL = ("s_branch", "s_endpgm", "s_setpc_b64")


def sgprs(tok):
    """The SGPR names an operand token covers (s7, s[4:5], m0, vcc)."""
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    if re.fullmatch(r"s\d+|m0", tok):
        return {tok}
    if tok in ("vcc", "vcc_lo", "vcc_hi"):
        return set(VCC) if tok == "vcc" else {VCC[0] if tok == "vcc_lo" else VCC[1]}
    return set()


def _split(ins):
    parts = ins.replace(",", " ").split()
    return parts[0], parts[1:]


def valu_writes(ins):
    """SGPRs (and M0) a VALU instruction writes."""
    op, args = _split(ins)
    base = re.sub(r"_e(32|64)$", "", op)
    out = sgprs(args[0]) if args else set()
    if base in _CARRY_OPS or base.startswith(("v_cmp_", "v_cmps_")):
        if op.endswith("_e64") and base in _CARRY_OPS and len(args) > 1:
            out |= sgprs(args[1])
        elif not op.endswith("_e64"):
            out |= set(VCC)  # VOP2/VOPC forms write VCC implicitly
    return out


def _wait_states(ins):
    op, args = _split(ins)
    return int(args[0], 0) + 1 if op == "s_nop" else 1


def functions(asm):
    """(name, items) per function of an assembly listing; an item is
    ("L", label) or ("I", instruction text)."""
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.find(".Lfunc_end", m.start())
        items = []
        for line in asm[m.start():end].splitlines()[1:]:
            line = line.split(";")[0].strip()
            if not line or line.startswith("."):
                if re.fullmatch(r"\.LBB\d+_\d+:", line):
                    items.append(("L", line[:-1]))
                continue
            if line.endswith(":"):
                items.append(("L", line[:-1]))
            else:
                items.append(("I", line))
        yield m.group(1), items


def hazards(asm):
    """Violations of the two rules in one assembly listing, and the number of
    LDS-DMA loads seen. The look-back follows control flow: at a label it
    continues through the fall-through predecessor (unless that ends in an
    unconditional branch) and through every branch to the label."""
    bad, loads = [], 0
    for name, items in functions(asm):
        branches_to = {}
        for i, (kind, text) in enumerate(items):
            if kind == "I" and text.startswith(("s_cbranch", "s_branch")):
                branches_to.setdefault(text.split()[-1], []).append(i)

        def walk(j, waited, reads, load, seen):
            # instructions at j, j-1, ... with `waited` wait states already between them and the load
            while j >= 0 and waited < VMEM_SGPR_WAIT:
                kind, text = items[j]
                if kind == "L":
                    key = (j, waited)
                    if key in seen:
                        return
                    seen.add(key)
                    for b in branches_to.get(text, ()):
                        walk(b, waited, reads, load, seen)
                    prev = items[j - 1] if j > 0 else None
                    if prev is not None and prev[0] == "I" and prev[1].startswith(_UNCONDITIONAL):
                        return
                    j -= 1
                    continue
                op, args = _split(text)
                if op.startswith("v_"):
                    hit = valu_writes(text) & reads
                    if hit:
                        bad.append(f"{name}: {text} {waited} wait states before {load}")
                elif op.startswith("s_") and args and "m0" in sgprs(args[0]) and waited < M0_LDS_DMA_WAIT:
                    bad.append(f"{name}: {text} {waited} wait states before {load}")
                waited += _wait_states(text)
                j -= 1

        for i, (kind, text) in enumerate(items):
            if kind != "I":
                continue
            op, args = _split(text)
            if op.startswith("v_") and "m0" in valu_writes(text):
                bad.append(f"{name}: VALU writes M0: {text}")
            if not op.startswith("global_load_lds"):
                continue
            loads += 1
            reads = (sgprs(args[1]) if len(args) > 1 else set()) | {"m0"}
            walk(i - 1, 0, reads, text, set())
    return bad, loads


def sources_with_lds_dma(csrc, sources):
    out = []
    for s in sources:
        text = open(os.path.join(csrc, s)).read()
        if "lds_load16(" in text or "lds_load4(" in text:
            out.append(s)
    return out


def device_asm(hipcc, flags, csrc, src, out_path):
    """The gfx950 assembly of one source, compiled with the library's flags."""
    cmd = [hipcc, *flags, "-I", csrc, "--cuda-device-only", "-S", os.path.join(csrc, src), "-o", out_path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stdout}\n{r.stderr}")
    with open(out_path) as f:
        return f.read()
