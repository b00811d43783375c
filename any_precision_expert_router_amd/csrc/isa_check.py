"""Build-time checks of the generated gfx950 assembly.

The activation broadcast uses hand-written DPP dot products (v_dot2c_f32_f16_dpp
row_newbcast) in inline assembly, which the compiler's hazard recognizer does not see.  The
rules checked, each as a minimum number of wait states between two instructions:
  * VALU writes a VGPR -> a DPP instruction reads it (any operand, the accumulator of the "c"
    forms included): 2;
  * EXEC written -> a DPP instruction: 5;
  * a DOT instruction writes a VGPR -> any other instruction reads it: 3 (the same DOT opcode
    may take it back as its accumulator at once).
`check` walks back from every reading instruction along every control-flow path (fall-through
and branches into its block) and reports each gap that is too short.

`scratch_users` reports kernels that use scratch memory (register spills).

`flat_accesses` reports flat (generic address) memory instructions.  A flat load may go to LDS or
to global memory, so its result needs a wait for every vector load in flight (vmcnt(0)), which
drains the streaming ring; every access in these kernels must name its address space.
"""
from __future__ import annotations

import re
import sys

DPP_VGPR_WAITS = 2
DPP_EXEC_WAITS = 5
DOT_RESULT_WAITS = 3
_STORES = ("global_store", "buffer_store", "flat_store", "scratch_store", "ds_write", "ds_store")


def _regs(tok: str):
    tok = tok.strip()
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _program(path: str):
    """[(kind, text)] with kind 'label' or 'inst', in listing order."""
    out = []
    with open(path) as f:
        for line in f:
            s = line.split(";")[0].strip()
            if not s or s.startswith("."):
                if s.startswith(".LBB") and s.endswith(":"):
                    out.append(("label", s[:-1]))
                continue
            if s.endswith(":"):
                out.append(("label", s[:-1]))
            else:
                out.append(("inst", s))
    return out


def _operands(inst: str):
    parts = inst.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip() for o in parts[1].split(",")]


def _vgpr_writes(inst: str):
    """VGPRs written by a VALU instruction (its first operand), else empty."""
    if not inst.startswith("v_") or inst.startswith(("v_readlane", "v_readfirstlane", "v_cmp_", "v_cmpx_")):
        return set()
    ops = _operands(inst)
    return _regs(ops[0]) if ops else set()


def _writes_exec(inst: str):
    ops = _operands(inst)
    return bool(ops) and (ops[0].startswith("exec") or inst.startswith("v_cmpx"))


def _is_dot(inst: str) -> bool:
    return inst.startswith("v_dot")


def _reads(inst: str):
    """(VGPRs read, VGPRs read only as the accumulator of a DOT "c" form)."""
    ops = _operands(inst)
    op = inst.split()[0]
    if not ops:
        return set(), set()
    if op.startswith(_STORES) or op.startswith(("s_", "buffer_atomic", "global_atomic")):
        srcs = ops
    else:
        srcs = ops[1:]
    reads = set()
    for o in srcs:
        reads |= _regs(o)
    acc = set()
    if _is_dot(op) and op.split("_dpp")[0].endswith("c_f32_f16"):   # accumulating form: vdst is read
        acc = _regs(ops[0])
    elif op.startswith(("v_fmac", "v_mac")):
        reads |= _regs(ops[0])
    return reads | acc, acc


def check(path: str):
    """Return (number of DPP instructions, list of hazard descriptions)."""
    prog = _program(path)
    label_at = {t: i for i, (k, t) in enumerate(prog) if k == "label"}
    preds = {}  # label -> indices of branch instructions that jump to it
    for i, (k, t) in enumerate(prog):
        if k == "inst" and t.startswith(("s_branch", "s_cbranch")):
            tgt = t.split()[-1]
            if tgt in label_at:
                preds.setdefault(tgt, []).append(i)
    problems = []
    horizon = max(DPP_EXEC_WAITS, DOT_RESULT_WAITS)

    def walk(start, target, is_dpp, reads, acc_only, waits, seen):
        op = target.split()[0]
        j = start
        while j >= 0:
            kind, t = prog[j]
            if kind == "label":
                for b in preds.get(t, []):
                    if (b, waits) not in seen:
                        seen.add((b, waits))
                        walk(b - 1, target, is_dpp, reads, acc_only, waits + 1, seen)
                j -= 1
                if j >= 0 and prog[j][0] == "inst" and prog[j][1].startswith("s_branch"):
                    return  # no fall-through into this label
                continue
            if t.startswith("s_endpgm"):
                return
            if t.startswith("s_nop"):
                waits += int(t.split()[1], 0) + 1
            else:
                w = _vgpr_writes(t)
                if is_dpp and waits < DPP_EXEC_WAITS and _writes_exec(t):
                    problems.append(f"EXEC write {t!r} -> {target!r} ({waits} wait states)")
                if is_dpp and waits < DPP_VGPR_WAITS and w & reads:
                    problems.append(f"VGPR write {t!r} -> DPP {target!r} ({waits} wait states)")
                if _is_dot(t) and waits < DOT_RESULT_WAITS and w & reads:
                    same_as_acc = t.split()[0] == op and not (w & (reads - acc_only))
                    if not same_as_acc:
                        problems.append(f"DOT result {t!r} -> {target!r} ({waits} wait states)")
                waits += 1
            if waits >= horizon:
                return
            j -= 1

    n = 0
    for i, (kind, t) in enumerate(prog):
        if kind != "inst":
            continue
        op = t.split()[0]
        is_dpp = op.startswith("v_") and "_dpp" in op
        n += is_dpp
        if not (op.startswith(("v_", "ds_", "global_", "buffer_", "flat_"))):
            continue
        reads, acc_only = _reads(t)
        if reads:
            walk(i - 1, t, is_dpp, reads, acc_only, 0, set())
    return n, problems


def scratch_users(path: str):
    """Names of the kernels in the assembly whose private segment (scratch) is not empty."""
    out, name = [], None
    with open(path) as f:
        for line in f:
            m = re.match(r"\s*\.amdhsa_kernel\s+(\S+)", line)
            if m:
                name = m.group(1)
            m = re.match(r"\s*\.amdhsa_private_segment_fixed_size\s+(\d+)", line)
            if m and name and int(m.group(1)) > 0:
                out.append(f"{name} ({m.group(1)} bytes)")
    return out


def flat_accesses(path: str):
    return [t for kind, t in _program(path) if kind == "inst" and t.startswith("flat_")]


if __name__ == "__main__":
    bad = False
    for p in sys.argv[1:]:
        n, probs = check(p)
        print(f"{p}: {n} DPP instructions, {len(probs)} hazards")
        for q in probs[:20]:
            print("  " + q)
        bad |= bool(probs)
    sys.exit(1 if bad else 0)
