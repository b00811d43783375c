"""Build-time check of the generated gfx950 assembly.

The activation broadcast uses hand-written DPP (v_dot2c_f32_f16_dpp row_newbcast) in inline
assembly, which the compiler's hazard recognizer does not see.  The ISA requires two wait states
between a VALU write of a VGPR and a DPP read of it, and five between an EXEC write and a DPP
instruction.  This scans every DPP instruction of the device assembly and fails the build if
either gap is shorter.
"""
from __future__ import annotations

import re
import sys


def _regs(tok: str):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _instructions(path: str):
    with open(path) as f:
        lines = [l.strip() for l in f]
    return [l.split(";")[0].strip() for l in lines
            if l and not l.startswith((";", ".")) and not l.endswith(":")]


def check(path: str):
    """Return (number of DPP instructions, list of hazard descriptions)."""
    insts = _instructions(path)
    problems = []
    n = 0
    for i, ins in enumerate(insts):
        if not ins.startswith("v_") or "_dpp" not in ins.split()[0]:
            continue
        n += 1
        src0 = _regs([o.strip() for o in ins.split(None, 1)[1].split(",")][1])
        waits = 0
        for j in range(i - 1, max(-1, i - 8), -1):
            prev = insts[j]
            if prev.startswith("s_nop"):
                waits += int(prev.split()[1], 0) + 1
                if waits >= 5:
                    break
                continue
            first = prev.split(",")[0]
            if (" exec" in first or prev.startswith("v_cmpx")) and waits < 5:
                problems.append(f"EXEC write {prev!r} -> {ins!r}")
            if prev.startswith("v_") and not prev.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
                dst = _regs(first.split(None, 1)[1].strip()) if " " in first else set()
                if dst & src0 and waits < 2:
                    problems.append(f"VGPR write {prev!r} -> {ins!r}")
            waits += 1
            if waits >= 5:
                break
    return n, problems


if __name__ == "__main__":
    bad = False
    for p in sys.argv[1:]:
        n, probs = check(p)
        print(f"{p}: {n} DPP instructions, {len(probs)} hazards")
        for q in probs[:20]:
            print("  " + q)
        bad |= bool(probs)
    sys.exit(1 if bad else 0)
