"""Check of compiled gfx950 assembly for DPP data hazards.

On gfx9 a VALU instruction with a DPP source must not read a VGPR that was
written in the two preceding wait states (an instruction is one wait state,
``s_nop N`` is N + 1), and must not follow a VALU write of EXEC by fewer than
five.  The compiler inserts these wait states for the DPP instructions it
generates, but not around inline assembly, which the kernels use for
``v_fmac_f32_dpp``.  ``check_asm`` walks every DPP instruction of a device
assembly file backwards through its basic block and, at the block start,
through every predecessor block, and reports each place where a write comes
too close.  The rule applied is the conservative one: every VGPR operand the
DPP instruction reads (the DPP source, the other source and a tied
accumulator), and a write by any instruction.

``__graft_entry__.build`` runs it on the assembly of the library it builds
and fails the build on any finding.
"""
from __future__ import annotations

import re
import sys
from dataclasses import dataclass, field

VGPR_WAIT = 2
EXEC_WAIT = 5

_LABEL = re.compile(r"^([.\w$]+):")
_VREG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")
_TERMINATORS_NO_FALLTHROUGH = ("s_branch", "s_endpgm", "s_setpc_b64", "s_trap")


@dataclass
class Instr:
    op: str
    args: str
    line: int

    @property
    def wait_states(self) -> int:
        if self.op == "s_nop":
            return int(self.args.split()[0], 0) + 1
        return 1


@dataclass
class Block:
    label: str
    instrs: list = field(default_factory=list)
    succs: list = field(default_factory=list)
    preds: list = field(default_factory=list)


def _regs(text: str) -> set:
    out = set()
    for m in _VREG.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _operands(args: str) -> list:
    # operands are comma separated; modifiers (row_newbcast:3, offen, ...) follow the last one after a space
    parts = [p.strip() for p in args.split(",")]
    if parts:
        parts[-1] = parts[-1].split()[0] if parts[-1] else parts[-1]
    return [p for p in parts if p]


def vgpr_defs(ins: Instr) -> set:
    """VGPRs an instruction writes (its vector destination operand(s))."""
    op = ins.op
    ops = _operands(ins.args)
    if not ops:
        return set()
    if op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
        return set()  # scalar or condition destination
    if op.startswith("v_") or op.startswith(("ds_read", "ds_load", "buffer_load", "global_load", "flat_load",
                                            "scratch_load", "ds_bpermute", "ds_permute", "ds_swizzle")):
        if op.startswith("ds_") and not op.startswith(("ds_read", "ds_load", "ds_bpermute", "ds_permute",
                                                         "ds_swizzle")):
            return set()
        d = _regs(ops[0])
        if "swap" in op and len(ops) > 1:
            d |= _regs(ops[1])
        return d
    return set()


def writes_exec(ins: Instr) -> bool:
    return ins.op.startswith("v_cmpx") or (ins.op.startswith("v_") and ins.args.startswith("exec"))


def is_dpp(ins: Instr) -> bool:
    return ins.op.endswith("_dpp") or bool(re.search(r"\b(row_\w+|quad_perm|wave_\w+):", ins.args))


def vgpr_uses(ins: Instr) -> set:
    ops = _operands(ins.args)
    uses = set()
    for o in ops[1:]:
        uses |= _regs(o)
    if re.match(r"v_(fmac|mac)_", ins.op):
        uses |= _regs(ops[0])  # tied accumulator
    return uses


def parse_functions(text: str) -> dict:
    """function name -> list of basic blocks, with successor / predecessor labels."""
    funcs = {}
    cur_fn = None
    blocks = None
    for ln, raw in enumerate(text.splitlines(), 1):
        line = raw.split(";")[0].rstrip()
        if not line.strip():
            continue
        m = _LABEL.match(line)
        if m:
            name = m.group(1)
            if name.startswith(".Lfunc_end"):
                cur_fn = None
                continue
            if not name.startswith("."):
                cur_fn = name
                blocks = [Block(name)]
                funcs[name] = blocks
            elif cur_fn is not None:
                blocks.append(Block(name))
            continue
        if cur_fn is None:
            continue
        s = line.strip()
        if s.startswith("."):
            continue
        parts = s.split(None, 1)
        ins = Instr(parts[0], parts[1] if len(parts) > 1 else "", ln)
        blocks[-1].instrs.append(ins)
        if ins.op.startswith("s_cbranch") or ins.op.startswith(_TERMINATORS_NO_FALLTHROUGH):
            # a branch ends the block; what follows (printed without a label) is the fall-through block
            blocks.append(Block(f"{cur_fn}+{ln}"))
    for blocks in funcs.values():
        index = {b.label: i for i, b in enumerate(blocks)}
        for i, b in enumerate(blocks):
            fall = True
            for ins in b.instrs:
                if ins.op.startswith("s_cbranch") or ins.op == "s_branch":
                    tgt = ins.args.split()[0]
                    if tgt in index:
                        b.succs.append(tgt)
            if b.instrs and b.instrs[-1].op.startswith(_TERMINATORS_NO_FALLTHROUGH):
                fall = False
            if fall and i + 1 < len(blocks):
                b.succs.append(blocks[i + 1].label)
        for b in blocks:
            for s in b.succs:
                blocks[index[s]].preds.append(b.label)
    return funcs


def _scan_back(blocks, index, bi, pos, uses, dpp, findings, fn):
    # (block index, position to start before, wait states so far); explore all paths until both limits are met
    seen = set()
    stack = [(bi, pos, 0)]
    while stack:
        b, p, ws = stack.pop()
        if (b, p, ws) in seen:
            continue
        seen.add((b, p, ws))
        instrs = blocks[b].instrs
        while p > 0 and ws < EXEC_WAIT:
            p -= 1
            ins = instrs[p]
            if ws < VGPR_WAIT and (vgpr_defs(ins) & uses):
                findings.append((fn, dpp.line, ins.line, f"{dpp.op} {dpp.args.split(' row_')[0]} reads "
                                 f"v{sorted(vgpr_defs(ins) & uses)} written {ws} wait state(s) earlier by "
                                 f"{ins.op} (line {ins.line})"))
            if writes_exec(ins):
                findings.append((fn, dpp.line, ins.line, f"{dpp.op} {ws} wait state(s) after an EXEC write by "
                                 f"{ins.op} (line {ins.line})"))
            ws += ins.wait_states
        if p == 0 and ws < EXEC_WAIT:
            for pl in blocks[b].preds:
                pi = index[pl]
                stack.append((pi, len(blocks[pi].instrs), ws))


def check_asm(text: str) -> list:
    """Findings (function, DPP line, writer line, message) for one assembly file."""
    findings = []
    for fn, blocks in parse_functions(text).items():
        index = {b.label: i for i, b in enumerate(blocks)}
        for bi, b in enumerate(blocks):
            for pos, ins in enumerate(b.instrs):
                if is_dpp(ins):
                    _scan_back(blocks, index, bi, pos, vgpr_uses(ins), ins, findings, fn)
    return findings


def count_dpp(text: str) -> int:
    return sum(1 for blocks in parse_functions(text).values() for b in blocks for i in b.instrs if is_dpp(i))


def main(paths) -> int:
    bad = 0
    for p in paths:
        text = open(p).read()
        f = check_asm(text)
        print(f"{p}: {count_dpp(text)} DPP instructions, {len(f)} hazards")
        for fn, _, _, msg in f[:20]:
            print(f"  {fn}: {msg}")
        bad += len(f)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
