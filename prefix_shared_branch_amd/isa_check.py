"""Build-time checks of the generated gfx950 ISA.

scan: fails the build if a vector-memory store of more than 8 bytes is followed, within two wait
states, by a VALU instruction that overwrites one of the store's data registers. The hardware
reads such store data after issue, so the store would write the new value; the compiler
covers this case for FLAT/global stores but not for buffer stores that use an SGPR offset.

loop_scratch: fails the build if a named kernel touches scratch memory inside a loop. In the
one-wave-per-SIMD dK/dV kernel a spill reload in the step loop waits for every direct load in
flight (vmcnt(0)) and costs most of its speed; its register assignment is tuned to avoid spills,
and a change elsewhere in the kernel can undo that without any other sign.
"""
from __future__ import annotations

import re

_STORE = re.compile(r"^\s*(buffer_store_dwordx[34]|global_store_dwordx[34]|flat_store_dwordx[34]|"
                     r"scratch_store_dwordx[34])\s+(.*)$")
_WAIT_STATES = 2


def _regs(spec: str) -> set[int]:
    spec = spec.strip()
    m = re.match(r"v\[(\d+):(\d+)\]$", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


def _parse(lines):
    """Instructions as (line number, text) plus a map from label to the index of the next instruction."""
    insts, labels = [], {}
    for n, raw in enumerate(lines):
        s = raw.split(";")[0].strip()
        if not s or s.startswith("."):
            if s.startswith(".LBB") and s.endswith(":"):
                labels[s[:-1]] = len(insts)
            continue
        if s.endswith(":"):
            labels[s[:-1]] = len(insts)
            continue
        insts.append((n, s))
    return insts, labels


def _hazard_after(insts, labels, k, data, waits, seen):
    """Follow every control path from instruction k on until _WAIT_STATES wait states have passed."""
    while k < len(insts) and waits < _WAIT_STATES:
        if (k, waits) in seen:
            return None
        seen.add((k, waits))
        n2, s2 = insts[k]
        op = s2.split()[0]
        if op == "s_endpgm":
            return None
        if op == "s_nop":
            waits += int(s2.split()[1], 0) + 1
            k += 1
            continue
        if op.startswith("s_branch") or op.startswith("s_cbranch"):
            target = s2.split()[1]
            if target in labels:
                hit = _hazard_after(insts, labels, labels[target], data, waits + 1, seen)
                if hit:
                    return hit
            if op.startswith("s_branch"):
                return None
            waits += 1
            k += 1
            continue
        if op.startswith("v_") and not op.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
            dst = s2.split(None, 1)[1].split(",")[0]
            if _regs(dst) & data:
                return f"'{s2}' (line {n2 + 1}) after {waits} wait state(s)"
        waits += 1
        k += 1
    return None


def scan(asm_text: str) -> list[str]:
    insts, labels = _parse(asm_text.splitlines())
    problems = []
    for k, (n, s) in enumerate(insts):
        m = _STORE.match(s)
        if not m:
            continue
        ops = [o.strip() for o in m.group(2).split(",")]
        data = _regs(ops[0] if m.group(1).startswith("buffer") else ops[1])
        hit = _hazard_after(insts, labels, k + 1, data, 0, set())
        if hit:
            problems.append(f"line {n + 1}: '{s}' then {hit}")
    return problems


# kernels whose loops must not touch scratch memory
LOOP_SCRATCH_FREE = ("replay_bwd_dkdv_w64",)


def loop_scratch(asm_text: str, kernels=LOOP_SCRATCH_FREE) -> list[str]:
    """Scratch accesses between a loop label and a later branch back to it, in the named kernels."""
    problems = []
    lines = asm_text.splitlines()
    starts = [(n, l.split(":")[0]) for n, l in enumerate(lines) if re.match(r"^_Z\S+:", l)]
    for i, (n0, name) in enumerate(starts):
        if not any(k in name for k in kernels):
            continue
        n1 = starts[i + 1][0] if i + 1 < len(starts) else len(lines)
        insts, labels = _parse(lines[n0:n1])
        for b, (_, s) in enumerate(insts):
            op = s.split()[0]
            if not (op.startswith("s_branch") or op.startswith("s_cbranch")):
                continue
            target = s.split()[1]
            if target in labels and labels[target] <= b:
                for k in range(labels[target], b + 1):
                    if insts[k][1].startswith("scratch_"):
                        problems.append(f"{name}: line {n0 + insts[k][0] + 1}: '{insts[k][1]}' inside a loop")
    return sorted(set(problems))
