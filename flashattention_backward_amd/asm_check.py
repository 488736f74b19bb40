"""Build-time check of the inline-asm MFMAs in the compiled device code.

The kernels issue some MFMAs through inline asm (to pin accumulators to AGPRs and to order
them against vector work), so the compiler's hazard recognizer does not protect their source
operands.  On gfx950 a VALU instruction (including v_accvgpr_read/write moves) that writes a
VGPR needs two wait states before an MFMA reads that register as SrcA, SrcB or SrcC.  This
module scans the gfx950 assembly for any MFMA with such a producer among the preceding
instructions that supply fewer than two wait states (an instruction is one wait state,
``s_nop N`` is N + 1).  The build fails if one is found.
"""
from __future__ import annotations

import re

WAIT_STATES = 2

_RANGE = re.compile(r"([va])\[(\d+):(\d+)\]$")
_SINGLE = re.compile(r"([va])(\d+)$")


def _regs(tok: str) -> set:
    tok = tok.strip()
    m = _RANGE.match(tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _SINGLE.match(tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _vector_dst(inst: str) -> set:
    """Registers written by a non-MFMA vector instruction (its first operand)."""
    op, _, rest = inst.partition(" ")
    if not op.startswith("v_") or op.startswith("v_mfma") or not rest:
        return set()
    if op.startswith("v_cmp") and op.endswith("_e32"):  # writes vcc only
        return set()
    return _regs(rest.split(",")[0])


def _instructions(asm: str) -> list:
    out = []
    for line in asm.splitlines():
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        out.append(re.sub(r"\s+", " ", s))
    return out


def mfma_operand_hazards(asm: str, wait_states: int = WAIT_STATES) -> list:
    """(producer, mfma) pairs where a vector write reaches an MFMA source too early."""
    insts = _instructions(asm)
    bad = []
    for i, inst in enumerate(insts):
        if not inst.startswith("v_mfma"):
            continue
        ops = inst.split(" ", 1)[1].split(",")
        srcs = set()
        for o in ops[1:4]:
            srcs |= _regs(o)
        ws, j = 0, i - 1
        while j >= 0 and ws < wait_states:
            prev = insts[j]
            if prev.startswith("s_nop"):
                ws += int(prev.split()[1], 0) + 1
            else:
                if _vector_dst(prev) & srcs:
                    bad.append((prev, inst))
                    break
                ws += 1
            j -= 1
    return bad


def count_mfma(asm: str) -> int:
    return sum(1 for s in _instructions(asm) if s.startswith("v_mfma"))
