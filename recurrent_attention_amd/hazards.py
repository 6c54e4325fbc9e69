"""Check gfx950 device assembly for matrix-core results read too early.

An MFMA writes its destination registers some cycles after it issues, and
the hardware does not stall a later VALU, LDS, memory or export
instruction that touches those registers: the program must put enough
independent instructions (wait states) in between.  The compiler pads
straight-line code, but a uniform branch between the MFMA and the first
reader has been seen to lose that padding, leaving the reader with the
accumulator's old value.  This module re-checks every path of the control
flow graph of each function in an assembly file (``hipcc --cuda-device-only
-S``), so a build can be rejected before it reaches a GPU.

``python -m recurrent_attention_amd.hazards FILE.s ...`` prints the
violations and exits non-zero when there are any.

Wait states required between an MFMA and the first non-MFMA instruction
that reads or writes one of its destination registers, for the MFMA opcodes
the kernels use.  They are the distances the compiler itself keeps in
straight-line code on gfx950: a 4-pass XDL operation needs passes + 4, the
16x16 fp32 operation (not XDL) needs 10.  An opcode missing from the table
is reported, so that a new instruction cannot pass unchecked.
"""
from __future__ import annotations

import re
import sys
from dataclasses import dataclass

REQUIRED_WAIT_STATES = {
    "v_mfma_f32_16x16x32_bf16": 8,
    "v_mfma_f32_16x16x16_bf16": 8,
    "v_mfma_f32_16x16x4_f32": 10,
}

_LABEL = re.compile(r"^([A-Za-z_.$][\w.$]*):")
_REG_RANGE = re.compile(r"\b([av])\[(\d+):(\d+)\]")
_REG_ONE = re.compile(r"\b([av])(\d+)\b")
_NOP = re.compile(r"^s_nop\s+(\d+)")


@dataclass
class Violation:
    function: str
    mfma: str
    reader: str
    wait_states: int
    required: int
    path: list

    def __str__(self):
        via = " -> ".join(p for p in self.path if p) or "straight line"
        return (f"{self.function}: '{self.reader}' is {self.wait_states} wait states after "
                f"'{self.mfma}' (needs {self.required}; path: {via})")


def registers(text: str) -> set:
    """VGPR/AGPR names ('v12', 'a3') that an operand string mentions."""
    out = set()
    for m in _REG_RANGE.finditer(text):
        out.update(f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1))
    text = _REG_RANGE.sub(" ", text)
    out.update(f"{m.group(1)}{m.group(2)}" for m in _REG_ONE.finditer(text))
    return out


def _operands(inst: str):
    parts = inst.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip() for o in parts[1].split(",")]


def _wait_states(inst: str) -> int:
    m = _NOP.match(inst)
    return int(m.group(1)) + 1 if m else 1


def functions(asm: str):
    """{function name: [('label', name) | ('inst', text)]} in layout order."""
    funcs, cur = {}, None
    for raw in asm.split("\n"):
        line = raw.split(";")[0].rstrip()
        if not line.strip():
            continue
        m = _LABEL.match(line)
        if m:
            name = m.group(1)
            if not name.startswith(".L"):
                cur = funcs.setdefault(name, [])
            elif cur is not None:
                cur.append(("label", name))
            continue
        if cur is None or not line[0].isspace():
            continue
        text = line.strip()
        if text.startswith("."):
            continue
        cur.append(("inst", text))
    return funcs


def _blocks(items):
    blocks = [[None, []]]
    for kind, x in items:
        if kind == "label":
            blocks.append([x, []])
            continue
        blocks[-1][1].append(x)
        op = x.split(None, 1)[0]
        if op.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc", "s_trap")):
            blocks.append([None, []])
    blocks = [b for b in blocks if b[0] is not None or b[1]]
    index = {b[0]: i for i, b in enumerate(blocks) if b[0] is not None}
    succ = []
    for i, (_, insts) in enumerate(blocks):
        last = insts[-1].split() if insts else [""]
        nxt = [i + 1] if i + 1 < len(blocks) else []
        if last[0] == "s_branch":
            s = [index.get(last[1])]
        elif last[0].startswith("s_cbranch"):
            s = [index.get(last[1].rstrip(","))] + nxt
        elif last[0].startswith(("s_endpgm", "s_setpc", "s_trap")):
            s = []
        else:
            s = nxt
        succ.append([j for j in s if j is not None])
    return blocks, succ


def check_function(name: str, items) -> list:
    blocks, succ = _blocks(items)
    found = []
    for bi, (_, insts) in enumerate(blocks):
        for ii, inst in enumerate(insts):
            op, ops = _operands(inst)
            if not op.startswith("v_mfma"):
                continue
            need = REQUIRED_WAIT_STATES.get(op)
            if need is None:
                found.append(Violation(name, inst, "(opcode missing from the table)", 0, 0, []))
                continue
            stack = [(bi, ii + 1, 0, (), frozenset(registers(ops[0])))]
            seen = set()
            while stack:
                b, i, w, path, dst = stack.pop()
                if w >= need or not dst or (b, i, w, dst) in seen:
                    continue
                seen.add((b, i, w, dst))
                body = blocks[b][1]
                if i >= len(body):
                    for s in succ[b]:
                        stack.append((s, 0, w, path + (blocks[s][0],), dst))
                    continue
                nxt = body[i]
                nop, nops = _operands(nxt)
                if nop.startswith("v_mfma"):
                    # a dependent MFMA whose accumulator input is exactly the
                    # earlier result is forwarded (and ordered) by the
                    # hardware; the result as a multiplicand, or a partial
                    # overlap of the accumulator, is not
                    src_ab = registers(",".join(nops[1:3])) if len(nops) >= 3 else set()
                    src_c = registers(nops[3]) if len(nops) >= 4 else set()
                    if (src_ab & dst) or ((src_c & dst) and src_c != dst):
                        found.append(Violation(name, inst, nxt, w, need, list(path)))
                        continue
                    # registers this MFMA rewrites now hold its result, whose
                    # readers are checked from this MFMA on
                    dst = dst - registers(nops[0])
                elif not nop.startswith("s_") and registers(",".join(nops)) & dst:
                    found.append(Violation(name, inst, nxt, w, need, list(path)))
                    continue
                stack.append((b, i + 1, w + _wait_states(nxt), path, dst))
    return found


def check_asm(asm: str) -> list:
    out = []
    for name, items in functions(asm).items():
        out.extend(check_function(name, items))
    return out


def main(argv=None):
    paths = sys.argv[1:] if argv is None else argv
    bad = 0
    for p in paths:
        with open(p) as f:
            vs = check_asm(f.read())
        for v in vs:
            print(f"{p}: {v}")
        bad += len(vs)
    print(f"{bad} violation(s) in {len(paths)} file(s)")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
