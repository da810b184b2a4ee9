"""A check of the library's inline assembly against a hazard the compiler does not cover.

The cross-entropy kernels issue their LDS-direct buffer loads as inline assembly.  The compiler
inserts the wait states the hardware needs between the instructions it generates, but it does not
look inside assembly blocks: a VALU instruction that writes an SGPR (v_readlane_b32 restoring a
spilled buffer descriptor, for one) followed by a vector memory instruction that reads that SGPR
needs five wait states, and with fewer the memory instruction can read a stale descriptor and
address memory that is not the buffer's.  hazards() lists every vector memory instruction inside
an assembly block that a VALU write of one of its SGPRs precedes by fewer than five wait states;
check() compiles sources to gfx950 assembly and runs it.  The build runs check() on the sources
that hold such assembly and refuses a library with any hazard.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

# sources whose kernels issue vector memory instructions from inline assembly
ASM_SOURCES = ["la_ce.hip"]
WAIT_STATES = 5


def _sgprs(tok: str) -> set:
    out = set()
    for a, b in re.findall(r"s\[(\d+):(\d+)\]", tok):
        out |= set(range(int(a), int(b) + 1))
    out |= {int(a) for a in re.findall(r"\bs(\d+)\b", tok)}
    return out


def _valu_sgpr_writes(ins: str) -> set:
    """SGPRs a VALU instruction writes: the destination of v_readlane / v_readfirstlane and of
    compares, and the scalar destinations of VOP3 forms (carry-outs)."""
    op, _, args = ins.partition(" ")
    if not op.startswith("v_"):
        return set()
    ops = [a.strip() for a in args.split(",")]
    if not ops:
        return set()
    if op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
        return _sgprs(ops[0])
    if op.endswith("_e64") or "_co_" in op:
        return _sgprs(ops[0]) | (_sgprs(ops[1]) if len(ops) > 1 else set())
    return set()


def hazards(asm: str) -> list:
    """The hazards in one assembly listing, as readable strings."""
    ins, in_asm = [], []
    inside = False
    for line in asm.splitlines():
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
            continue
        if t.startswith(";;#ASMEND"):
            inside = False
            continue
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        ins.append(t.split(";")[0].strip())
        in_asm.append(inside)
    found = []
    for k, t in enumerate(ins):
        m = re.match(r"(buffer_\w+|global_\w+|scratch_\w+)\s+\S+,\s+(s\[\d+:\d+\])", t)
        if not (m and in_asm[k]):
            continue
        reads = _sgprs(m.group(2))
        waits = 0
        for b in range(k - 1, max(-1, k - 4 * WAIT_STATES), -1):
            u = ins[b]
            if u.startswith("s_nop"):
                waits += int(u.split()[1], 0) + 1
            else:
                if _valu_sgpr_writes(u) & reads:
                    found.append(f"{waits} wait states: {u!r} -> {t!r}")
                    break
                waits += 1
            if waits >= WAIT_STATES:
                break
    return found


def check(hipcc: str, flags: list, csrc: str, sources=ASM_SOURCES) -> list:
    """Compiles each source to device assembly with the build's flags and returns its hazards."""
    found = []
    with tempfile.TemporaryDirectory() as tmp:
        for src in sources:
            out = os.path.join(tmp, src + ".s")
            subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", os.path.join(csrc, src), "-o", out],
                           check=True, capture_output=True)
            with open(out) as f:
                found += [f"{src}: {h}" for h in hazards(f.read())]
    return found
