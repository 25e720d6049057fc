"""Static check of gfx950 assembly for matrix-core products that accumulate onto the
result of a product of another shape too soon after it.

Measured on gfx950 (a one-wave probe with exact small-integer operands): when a
v_mfma_f32_16x16x16_bf16 takes as its accumulator (SrcC) the destination of a
v_mfma_f32_16x16x32_bf16 issued fewer than about five wait states earlier, or the
reverse, half of the accumulator elements are read before the first result is
written and the first product is lost there. Products of the same shape chain back
to back correctly. ROCm 7.2.0's compiler inserts no wait states for the mixed case,
so the kernels avoid it by construction and this check guards the generated code.

The check walks backwards from every MFMA with a register accumulator along every
path (fall-through and branches, so chains across a loop's back edge are seen),
counting wait states: s_nop N as N + 1, an intervening MFMA as 4 (its issue takes at
least four passes), any other instruction as 1. A path ends at an instruction that
writes the accumulator registers: an MFMA of another opcode reached with fewer than
MIN_WAIT wait states is reported.
"""
from __future__ import annotations

import re

MIN_WAIT = 6  # the probe needed 5 (s_nop 4); one more for margin

_REG = re.compile(r"^v\[(\d+):(\d+)\]$|^v(\d+)$")
_LABEL = re.compile(r"^(\.?[A-Za-z_][\w.$]*):")


def _regs(tok: str):
    m = _REG.match(tok.strip())
    if not m:
        return None
    if m.group(3) is not None:
        r = int(m.group(3))
        return set([r])
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def _operands(ins: str):
    op = ins.split()[0]
    return op, [a.strip() for a in ins[len(op):].split(",")]


def _functions(asm: str):
    """Yield (name, items) per function; items are ('label', name) or ('ins', text)."""
    name, items = None, []
    for raw in asm.splitlines():
        line = raw.split(";")[0].strip()
        if not line:
            continue
        m = _LABEL.match(line)
        if m and not line.startswith("."):  # a function symbol
            if name is not None:
                yield name, items
            name, items = m.group(1), []
            continue
        if name is None:
            continue
        if m:  # a local label such as .LBB3_12
            items.append(("label", m.group(1)))
            continue
        if line.startswith("."):  # directives
            continue
        items.append(("ins", line))
    if name is not None:
        yield name, items


def _cost(ins: str) -> int:
    if ins.startswith("s_nop"):
        return int(ins.split()[1], 0) + 1
    if ins.startswith("v_mfma"):
        return 4
    return 1


def check_function(items, min_wait: int = MIN_WAIT):
    """Violations in one function: (index, reader, writer, wait states)."""
    label_at = {it[1]: i for i, it in enumerate(items) if it[0] == "label"}
    # predecessors of each label: branches that target it, and fall-through
    branches_to = {}
    for i, (kind, text) in enumerate(items):
        if kind == "ins" and text.startswith(("s_branch", "s_cbranch")):
            tgt = text.split()[-1]
            branches_to.setdefault(tgt, []).append(i)

    def preds(i):
        """Instruction positions that can execute just before position i."""
        j = i - 1
        out = []
        while j >= 0 and items[j][0] == "label":
            out.extend(branches_to.get(items[j][1], []))
            j -= 1
        if j >= 0:
            kind, text = items[j]
            if not text.startswith(("s_branch", "s_endpgm", "s_setpc")):
                out.append(j)
        # a branch itself is a predecessor only of its target; a conditional branch
        # also falls through
        return out

    bad = []
    for i, (kind, text) in enumerate(items):
        if kind != "ins" or not text.startswith("v_mfma"):
            continue
        op, args = _operands(text)
        if len(args) < 4:
            continue
        acc = _regs(args[3])
        if not acc:
            continue
        seen = set()
        stack = [(p, 0) for p in preds(i)]
        while stack:
            p, wait = stack.pop()
            if (p, wait) in seen or wait >= min_wait:
                continue
            seen.add((p, wait))
            ptext = items[p][1]
            if ptext.startswith("v_mfma"):
                pop, pargs = _operands(ptext)
                dst = _regs(pargs[0])
                if dst and dst & acc:
                    if pop != op:
                        bad.append((i, text, ptext, wait))
                    continue  # this path's accumulator comes from here
            elif ptext.startswith(("v_", "ds_read", "global_load", "buffer_load", "flat_load", "scratch_load")):
                _, pargs = _operands(ptext)
                dst = _regs(pargs[0]) if pargs else None
                if dst and dst & acc:
                    continue  # written by a non-MFMA instruction: not a chain
            w = wait + _cost(ptext)
            for q in preds(p):
                stack.append((q, w))
    return bad


def check_asm(asm: str, min_wait: int = MIN_WAIT):
    """All violations in an assembly file: (function, reader, writer, wait states)."""
    out = []
    for name, items in _functions(asm):
        for _, reader, writer, wait in check_function(items, min_wait):
            out.append((name, reader, writer, wait))
    return out
