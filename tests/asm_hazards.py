"""Static check of the gfx950 assembly of the HIP sources for the issue hazards that hand-written
assembly hides from the compiler.

The compiler inserts the wait states that CDNA's hazard rules require between the instructions it
knows. It does not look inside inline assembly, so an MFMA or an M0 write issued from an `asm`
block is invisible to it: a later change of instruction order could put a dependent instruction
too close without any warning. This module parses the compiled assembly (`hipcc --cuda-device-only
-S`), builds each kernel's control-flow graph and checks, over every path, the distances (in wait
states: one per instruction, N + 1 for `s_nop N`) that these rules require:

* MFMA result -> any non-MFMA instruction that reads or writes one of its result registers:
  MFMA_RESULT_WAIT[opcode] wait states (the compiler's own figure: it puts `s_nop 11` between
  `v_mfma_f32_32x32x16_bf16` and a vector-ALU or memory read of its result).
* MFMA result -> another MFMA that reads it as an A or B operand, or as an accumulator it does not
  exactly overlap, or writes part of it: the same distance (conservative). Chains that accumulate
  in place (same opcode, accumulator = result, exact overlap) need none.
* MFMA accumulator input -> a later write of those registers by another instruction (the MFMA may
  still be reading them): the same distance (conservative).
* Vector-ALU write -> an MFMA that reads the register: VALU_TO_MFMA wait states (the compiler puts
  two between a vector-ALU write and an MFMA operand read).
* Scalar write of M0 -> an LDS DMA (`global_load_lds_*`), which takes its LDS address from M0:
  M0_TO_LDS_DMA wait state (the compiler puts `s_nop 0` there).

Every MFMA and every LDS DMA is checked, the compiler's as well as the hand-written ones, so the
compiler's own output also tests that these figures are not too strict.
"""
from __future__ import annotations

import re
from dataclasses import dataclass, field

MFMA_RESULT_WAIT = {"v_mfma_f32_32x32x16_bf16": 12}
VALU_TO_MFMA = 2
M0_TO_LDS_DMA = 1

_REG = re.compile(r"(?<![\w.])([vas])(?:\[(\d+):(\d+)\]|(\d+))(?![\w\[])")
_LABEL = re.compile(r"^([.\w$]+):")


@dataclass
class Instr:
    op: str
    operands: list[str]
    line: int  # 1-based line in the assembly text
    text: str

    @property
    def waits(self) -> int:
        if self.op == "s_nop":
            return int(self.operands[0], 0) + 1
        return 1

    def regs(self, which=None) -> set[tuple[str, int]]:
        ops = self.operands if which is None else [self.operands[i] for i in which
                                                   if i < len(self.operands)]
        out = set()
        for o in ops:
            for m in _REG.finditer(o):
                kind = m.group(1)
                if m.group(4) is not None:
                    out.add((kind, int(m.group(4))))
                else:
                    out.update((kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
        return out

    @property
    def is_mfma(self) -> bool:
        return self.op.startswith("v_mfma_")

    @property
    def is_valu(self) -> bool:
        return self.op.startswith("v_") and not self.is_mfma

    @property
    def is_lds_dma(self) -> bool:
        return self.op.startswith(("global_load_lds_", "scratch_load_lds_")) or (
            self.op.startswith("buffer_load_") and "lds" in self.operands[-1:])

    def vector_writes(self) -> set[tuple[str, int]]:
        """Vector or accumulation registers this instruction writes (first operand of a vector-ALU
        instruction or of a load that returns data to registers)."""
        if not self.operands:
            return set()
        returns = self.op.startswith(("ds_read", "ds_load", "global_load", "buffer_load",
                                      "flat_load", "scratch_load")) and not self.is_lds_dma
        if self.is_valu or self.is_mfma or returns:
            w = self.regs([0])
            if self.op.startswith("v_swap"):
                w |= self.regs([1])
            return {r for r in w if r[0] in "va"}
        return set()


@dataclass
class Block:
    label: str | None
    instrs: list[Instr] = field(default_factory=list)
    succ: list[int] = field(default_factory=list)
    pred: list[int] = field(default_factory=list)


@dataclass
class Function:
    name: str
    blocks: list[Block]


def _split_operands(rest: str) -> list[str]:
    # operands are comma separated; trailing modifiers (offset:16, sc1, cbsz:1 ...) are separated
    # by spaces after the last operand and are kept as further entries
    parts = [p.strip() for p in rest.split(",")] if rest.strip() else []
    if parts:
        last = parts[-1].split()
        parts = parts[:-1] + last
    return parts


def parse(text: str) -> list[Function]:
    """Split the assembly into functions (a symbol label up to its .Lfunc_end label) of basic
    blocks."""
    funcs: list[Function] = []
    cur: list[Block] | None = None
    name = None
    for ln, raw in enumerate(text.splitlines(), 1):
        line = raw.split(";")[0].split("//")[0].strip()
        if not line:
            continue
        m = _LABEL.match(line)
        if m:
            lab = m.group(1)
            if lab.startswith(".Lfunc_end"):
                cur = None
            elif not lab.startswith("."):  # a function symbol
                name, cur = lab, [Block(lab)]
                funcs.append(Function(name, cur))
            elif cur is not None and lab.startswith(".LBB"):
                cur.append(Block(lab))
            continue
        if cur is None or line.startswith("."):
            continue
        op, _, rest = line.partition(" ")
        ins = Instr(op, _split_operands(rest), ln, raw.strip())
        if cur[-1].instrs and cur[-1].instrs[-1].op.startswith(("s_branch", "s_cbranch",
                                                                "s_endpgm", "s_setpc")):
            cur.append(Block(None))
        cur[-1].instrs.append(ins)
    for f in funcs:
        index = {b.label: i for i, b in enumerate(f.blocks) if b.label}
        for i, b in enumerate(f.blocks):
            last = b.instrs[-1] if b.instrs else None
            falls = i + 1 < len(f.blocks)
            if last is not None and last.op == "s_branch":
                b.succ = [index[last.operands[0]]]
            elif last is not None and last.op.startswith("s_cbranch"):
                b.succ = [index[last.operands[0]]] + ([i + 1] if falls else [])
            elif last is not None and last.op in ("s_endpgm", "s_setpc_b64"):
                b.succ = []
            else:
                b.succ = [i + 1] if falls else []
        for i, b in enumerate(f.blocks):
            for s in b.succ:
                f.blocks[s].pred.append(i)
    return funcs


def _forward(f: Function, bi: int, ii: int, limit: int):
    """Yield (instr, wait states between the start instruction and it) for every instruction
    reachable within `limit` wait states after instruction ii of block bi."""
    best: dict[int, int] = {}
    stack = [(bi, ii + 1, 0)]
    while stack:
        b, i, w = stack.pop()
        blk = f.blocks[b]
        while i < len(blk.instrs) and w < limit:
            ins = blk.instrs[i]
            yield ins, w
            w += ins.waits
            i += 1
        if w < limit:
            for s in blk.succ:
                if best.get(s, limit) > w:
                    best[s] = w
                    stack.append((s, 0, w))


def _backward(f: Function, bi: int, ii: int, limit: int):
    """Yield (instr, wait states between it and the start instruction) for every instruction that
    can precede instruction ii of block bi within `limit` wait states."""
    best: dict[int, int] = {}
    stack = [(bi, ii - 1, 0)]
    while stack:
        b, i, w = stack.pop()
        blk = f.blocks[b]
        while i >= 0 and w < limit:
            ins = blk.instrs[i]
            yield ins, w
            w += ins.waits
            i -= 1
        if w < limit:
            for p in blk.pred:
                if best.get(p, limit) > w:
                    best[p] = w
                    stack.append((p, len(f.blocks[p].instrs) - 1, w))


def check(text: str) -> list[str]:
    """Every hazard found, one line each (function, line of the assembly, what)."""
    found = []
    for f in parse(text):
        for bi, blk in enumerate(f.blocks):
            for ii, ins in enumerate(blk.instrs):
                where = f"{f.name}: line {ins.line}: {ins.text}"
                if ins.is_mfma:
                    if ins.op not in MFMA_RESULT_WAIT:
                        found.append(f"{where}: no wait-state figure for {ins.op}")
                        continue
                    need = MFMA_RESULT_WAIT[ins.op]
                    dst = ins.regs([0])
                    acc = ins.regs([3]) - dst
                    for nxt, w in _forward(f, bi, ii, need):
                        if nxt.is_mfma:
                            chain = (nxt.op == ins.op and nxt.regs([0]) == dst
                                     and nxt.regs([3]) == dst)
                            touched = nxt.regs([1, 2]) & dst or (
                                not chain and (nxt.regs([0]) | nxt.regs([3])) & dst)
                            if touched:
                                found.append(f"{where}: MFMA result used by MFMA at line "
                                             f"{nxt.line} after {w} wait states (< {need})")
                        elif nxt.regs() & dst:
                            found.append(f"{where}: result accessed at line {nxt.line} "
                                         f"({nxt.text}) after {w} wait states (< {need})")
                        elif acc and nxt.vector_writes() & acc:
                            found.append(f"{where}: accumulator input overwritten at line "
                                         f"{nxt.line} after {w} wait states (< {need})")
                    srcs = ins.regs([1, 2, 3])
                    for prv, w in _backward(f, bi, ii, VALU_TO_MFMA):
                        if prv.is_valu and prv.vector_writes() & srcs:
                            found.append(f"{where}: operand written by the vector ALU at line "
                                         f"{prv.line} ({prv.text}) {w} wait states before "
                                         f"(< {VALU_TO_MFMA})")
                if ins.is_lds_dma:
                    for prv, w in _backward(f, bi, ii, M0_TO_LDS_DMA):
                        if prv.op.startswith("s_") and prv.operands[:1] == ["m0"]:
                            found.append(f"{where}: M0 written at line {prv.line} "
                                         f"({prv.text}) {w} wait states before "
                                         f"(< {M0_TO_LDS_DMA})")
    return found
