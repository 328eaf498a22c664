"""Wait-state check of the matrix-core instructions in a gfx950 assembly file.

The GEMM kernels issue their MFMAs as inline assembly, so the compiler does
not know them for what they are and inserts none of the wait states that the
CDNA3/CDNA4 instruction set requires around them.  The kernels are written so
that none are needed (every MFMA sits in the main loop; accumulators are
touched by other instructions only before the loop, behind an explicit drain,
and after it, behind another); this module checks that the compiled code
really has that shape.  It runs on the ``-save-temps`` assembly that the build
keeps, and the build fails on any finding.

Rules (in wait states: one per instruction, n + 1 for ``s_nop n``):

* a non-MFMA instruction that reads or writes a register an MFMA wrote must
  come at least ``RESULT_WAIT`` wait states after that MFMA (the longest
  XDL-result latency of the 16-pass forms plus two);
* an MFMA that reads a register as its A or B operand must come at least
  ``RESULT_WAIT`` after an MFMA that wrote it; an MFMA whose C operand
  overlaps an earlier MFMA's result without being the same register range
  likewise;
* a VALU instruction that writes a register an MFMA reads must come at least
  ``VALU_TO_MFMA`` wait states before it;
* no instruction may read or write the destination registers of a vector
  memory load before an ``s_waitcnt vmcnt(n)`` has retired that load (vector
  memory operations retire in issue order; a load that writes the matrix
  accumulators straight from memory is inline assembly too, so the compiler
  does not wait for it).

* ``m0`` belongs to the global -> LDS copies: it may appear only as the
  destination of an ``s_mov_b32`` that is directly followed by a
  ``buffer_load ... lds``.  The copies' inline assembly sets it and declares
  it clobbered, but the compiler treats m0 as reserved and does not promise to
  honour that, so no compiler-generated instruction may depend on it.

Control flow: the file is walked in order, and for every branch the last
instructions before it are also checked against the first instructions at its
target, so a loop's back edge and a forward jump are covered too.
"""
from __future__ import annotations

import re
import sys
from typing import Iterable, List, Optional, Set, Tuple

RESULT_WAIT = 18
VALU_TO_MFMA = 2

Reg = Tuple[str, int]
_RANGE = re.compile(r"^([va])\[(\d+):(\d+)\]$")
_SINGLE = re.compile(r"^([va])(\d+)$")
_KERNEL = re.compile(r"^(\S+):\s*(;.*)?$")
_LABEL = re.compile(r"^(\.LBB\w+):")
_BRANCH = re.compile(r"^s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)")


def regs(tok: str) -> Set[Reg]:
    tok = tok.strip()
    m = _RANGE.match(tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _SINGLE.match(tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


class Instr:
    __slots__ = ("op", "args", "text", "line")

    def __init__(self, op: str, args: List[str], text: str, line: int):
        self.op, self.args, self.text, self.line = op, args, text, line

    @property
    def is_mfma(self) -> bool:
        return self.op.startswith("v_mfma")

    @property
    def waits(self) -> int:
        return int(self.args[0], 0) + 1 if self.op == "s_nop" else 1

    def touched(self) -> Set[Reg]:
        if self.op.startswith("s_"):
            return set()
        out: Set[Reg] = set()
        for a in self.args:
            out |= regs(a)
        return out


def _parse(line: str, no: int) -> Optional[Instr]:
    s = line.split(";")[0].strip()
    if not s or s.startswith(".") or s.endswith(":"):
        return None
    parts = s.split(None, 1)
    args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
    return Instr(parts[0], args, s, no)


_VMEM = ("global_", "buffer_", "flat_", "scratch_")
_VMCNT = re.compile(r"vmcnt\((\d+)\)")


def _vmem_dest(ins: Instr) -> Optional[Set[Reg]]:
    """Registers a vector memory instruction writes when it returns (None
    for an instruction that is not vector memory)."""
    if not ins.op.startswith(_VMEM):
        return None
    if "_load" not in ins.op and "_atomic" not in ins.op:
        return set()  # stores write no register
    if "lds" in ins.args[-1].split() or ins.op.endswith("_lds_dword"):
        return set()  # global -> LDS: the first operand is an address
    if "_atomic" in ins.op and "glc" not in ins.text.split():
        return set()  # atomics without return
    return regs(ins.args[0])


def check_sequence(seq: Iterable[Instr]) -> List[str]:
    """Findings in one straight-line sequence of instructions."""
    found: List[str] = []
    recent: List[Tuple[Set[Reg], int, Instr]] = []   # MFMA results in flight: (regs, age, mfma)
    valu: List[Tuple[Set[Reg], int, Instr]] = []     # recent VALU writes: (regs, age, instr)
    loads: List[Tuple[Set[Reg], Instr]] = []         # vector memory in flight, oldest first
    for ins in seq:
        if ins.op == "s_waitcnt":
            m = _VMCNT.search(ins.text)
            if m:
                keep = int(m.group(1))
                loads = loads[len(loads) - keep:] if keep < len(loads) else loads
                if keep == 0:
                    loads = []
        t_all = ins.touched()
        for (r, ld) in loads:
            if r & t_all:
                found.append("line %d: %r touches the destination of %r before a wait retires it"
                             % (ins.line, ins.text, ld.text))
        dest = _vmem_dest(ins)
        if dest is not None:
            loads.append((dest, ins))
        if ins.is_mfma:
            dst = regs(ins.args[0])
            ab = regs(ins.args[1]) | regs(ins.args[2])
            c = regs(ins.args[3]) if len(ins.args) > 3 else set()
            for (r, age, w) in valu:
                if r & (ab | c) and age < VALU_TO_MFMA:
                    found.append("line %d: VALU write %r then MFMA %r after %d wait states"
                                 % (ins.line, w.text, ins.text, age))
            for (r, age, w) in recent:
                if r & ab:
                    found.append("line %d: MFMA operand from MFMA %r in flight (%d wait states)"
                                 % (ins.line, w.text, age))
                elif r & c and r != c:
                    found.append("line %d: MFMA C operand partly overlaps MFMA %r in flight (%d wait states)"
                                 % (ins.line, w.text, age))
            step = ins.waits
            recent = [(r, a + step, w) for (r, a, w) in recent if a + step < RESULT_WAIT]
            valu = [(r, a + step, w) for (r, a, w) in valu if a + step < VALU_TO_MFMA]
            recent.append((dst, 0, ins))
            continue
        t = ins.touched()
        for (r, age, w) in recent:
            if r & t:
                found.append("line %d: %r touches the result of MFMA %r after %d wait states"
                             % (ins.line, ins.text, w.text, age))
        step = ins.waits
        recent = [(r, a + step, w) for (r, a, w) in recent if a + step < RESULT_WAIT]
        valu = [(r, a + step, w) for (r, a, w) in valu if a + step < VALU_TO_MFMA]
        if ins.op.startswith("v_") and ins.args:
            valu.append((regs(ins.args[0]), 0, ins))
    return found


def _window(instrs: List[Instr], end: int, forward: bool) -> List[Instr]:
    """Instructions covering RESULT_WAIT wait states before index `end`
    (exclusive) or from index `end` on."""
    out: List[Instr] = []
    ws = 0
    i = end if forward else end - 1
    while 0 <= i < len(instrs) and ws < RESULT_WAIT + 2:
        out.append(instrs[i])
        ws += instrs[i].waits
        i += 1 if forward else -1
    return out if forward else out[::-1]


def check_kernel(body: List[Tuple[int, str]]) -> List[str]:
    instrs: List[Instr] = []
    labels = {}
    branches = []
    for no, line in body:
        s = line.strip()
        m = _LABEL.match(s)
        if m:
            labels[m.group(1)] = len(instrs)
            continue
        ins = _parse(line, no)
        if ins is None:
            continue
        b = _BRANCH.match(ins.text)
        if b:
            branches.append((len(instrs), b.group(1)))
        instrs.append(ins)
    found = check_sequence(instrs)
    for k, ins in enumerate(instrs):
        if not any(a == "m0" for a in ins.args):
            continue
        nxt = instrs[k + 1] if k + 1 < len(instrs) else None
        ok = (ins.op == "s_mov_b32" and ins.args[0] == "m0" and nxt is not None and
              nxt.op.startswith("buffer_load") and "lds" in nxt.args[-1].split())
        if not ok:
            found.append("line %d: %r uses m0 outside a global -> LDS copy" % (ins.line, ins.text))
    for at, target in branches:
        if target in labels:
            found += check_sequence(_window(instrs, at + 1, False) + _window(instrs, labels[target], True))
    return sorted(set(found))


def check_file(path: str, kernel_filter: str = "") -> dict:
    """{kernel symbol: [findings]} for every kernel in the file whose name
    contains `kernel_filter`."""
    lines = open(path).read().splitlines()
    out = {}
    cur = None
    body: List[Tuple[int, str]] = []
    for no, line in enumerate(lines, 1):
        m = _KERNEL.match(line)
        if m and not line.startswith(".") and not line.startswith(" ") and not line.startswith("\t"):
            if cur is not None:
                out[cur] = check_kernel(body)
            cur = m.group(1) if kernel_filter in m.group(1) else None
            body = []
            continue
        if cur is None:
            continue
        if "s_endpgm" in line:
            out[cur] = check_kernel(body)
            cur = None
            continue
        body.append((no, line))
    return out


def mfma_count(path: str) -> int:
    return sum(1 for line in open(path) if line.strip().startswith("v_mfma"))


def main(argv: List[str]) -> int:
    res = check_file(argv[1])
    bad = {k: v for k, v in res.items() if v}
    for k, v in bad.items():
        print(k)
        for f in v[:10]:
            print("   ", f)
    print("%d kernels checked, %d with findings" % (len(res), len(bad)))
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
