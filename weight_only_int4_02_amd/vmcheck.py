"""In-flight load registers: a check of the compiled kernels' gfx9 assembly.

The kernels issue most of their global loads as inline assembly and wait for
them with explicit `s_waitcnt vmcnt(N)`, so the compiler does not know a load
is still in flight.  If it copies, moves or reuses a destination register of
such a load before the wait that completes it (a live-range split into an
AGPR, a spill, a register reused for a temporary), the copy holds stale data
and the load later overwrites whatever the register holds then.  Neither is
visible in the compiler's resource-usage remarks: an AGPR copy is not a spill.

This module models the vector-memory counter over each kernel's control-flow
graph.  The pending loads are a queue, oldest first.  Every vector-memory
instruction (load, store, buffer-to-LDS copy) enters it; `s_waitcnt vmcnt(N)`
keeps only the newest N.  Where control flow merges, the queues are aligned at
their newest end and only what both hold is kept: the analysis finds what is
pending on every path (it reports no hazard that a path-insensitive merge
would invent, and may miss one that exists on some paths only).  An
instruction that names a register of a load still pending is reported, the
next load into that register included.
"""
from __future__ import annotations

import re
import subprocess
from typing import Dict, FrozenSet, List, Optional, Sequence, Tuple

_REG_RANGE = re.compile(r"^([va])\[(\d+):(\d+)\]")
_REG_ONE = re.compile(r"^([va])(\d+)\b")
_VMCNT = re.compile(r"vmcnt\((\d+)\)")
_LABEL = re.compile(r"^(\.?[\w.$]+):")
_FUNC = re.compile(r"^(_Z\w+):")
_MAX_PENDING = 63

Reg = Tuple[str, int]
Queue = Tuple[FrozenSet[Reg], ...]


def _regs(tok: str) -> FrozenSet[Reg]:
    tok = tok.strip()
    m = _REG_RANGE.match(tok)
    if m:
        return frozenset((m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1))
    m = _REG_ONE.match(tok)
    if m:
        return frozenset({(m.group(1), int(m.group(2)))})
    return frozenset()


def _strip(line: str) -> str:
    for c in (";", "//"):
        k = line.find(c)
        if k >= 0:
            line = line[:k]
    return line.strip()


def _operands(text: str) -> List[FrozenSet[Reg]]:
    """Register sets of the comma-separated operands, in order (modifiers
    after an operand, such as `offen` or `op_sel:[...]`, name none)."""
    return [_regs(p.strip().split(" ")[0]) if p.strip() else frozenset() for p in text.split(",")]


class _Instr:
    __slots__ = ("text", "op", "ops", "line")

    def __init__(self, text: str, line: int):
        self.text = text
        self.line = line
        parts = text.split(None, 1)
        self.op = parts[0]
        self.ops = _operands(parts[1]) if len(parts) > 1 else []


def _is_vmem(op: str) -> bool:
    return op.startswith(("buffer_", "global_", "flat_", "scratch_")) and not op.startswith(
        ("buffer_wbl2", "buffer_inv", "buffer_wbinvl1", "buffer_gl"))


def _is_load(ins: _Instr) -> bool:
    return "_load" in ins.op and " lds" not in ins.text and not ins.text.rstrip().endswith("lds")


def _blocks(body: Sequence[Tuple[int, str]]):
    """Basic blocks: (label or None, [instr], successor labels, falls through)."""
    blocks = []
    cur_label, cur = None, []

    def close(succ, falls):
        blocks.append([cur_label, cur, succ, falls])

    for line_no, raw in body:
        s = _strip(raw)
        if not s or s.startswith("."):
            m = _LABEL.match(s) if s else None
            if m and s.endswith(":"):
                if cur or cur_label is not None:
                    close([], True)
                cur_label, cur = m.group(1), []
            continue
        m = _LABEL.match(s)
        if m and s.endswith(":"):
            if cur or cur_label is not None:
                close([], True)
            cur_label, cur = m.group(1), []
            continue
        ins = _Instr(s, line_no)
        cur.append(ins)
        if ins.op == "s_branch":
            close([s.split()[1]], False)
            cur_label, cur = None, []
        elif ins.op.startswith("s_cbranch_"):
            close([s.split()[1]], True)
            cur_label, cur = None, []
        elif ins.op in ("s_endpgm", "s_setpc_b64"):
            close([], False)
            cur_label, cur = None, []
    if cur or cur_label is not None:
        close([], False)
    return blocks


def _join(a: Optional[Queue], b: Queue) -> Queue:
    # what is pending on every path into the block: the queues aligned at
    # their newest end, the common length, the registers common to both
    if a is None:
        return b
    n = min(len(a), len(b))
    return tuple(a[len(a) - k] & b[len(b) - k] for k in range(n, 0, -1))


def _step(q: Queue, ins: _Instr, report) -> Queue:
    if ins.op == "s_waitcnt":
        m = _VMCNT.search(ins.text)
        if m:
            keep = int(m.group(1))
            q = q[len(q) - keep:] if keep and len(q) > keep else (q if keep else ())
        return q
    live = frozenset().union(*q) if q else frozenset()
    used = frozenset().union(*ins.ops) if ins.ops else frozenset()
    if used & live and report is not None:
        report(ins, sorted(used & live))
    if _is_vmem(ins.op):
        dst = ins.ops[0] if (_is_load(ins) and ins.ops) else frozenset()
        q = (q + (dst,))[-_MAX_PENDING:]
    return q


def check_kernel(body: Sequence[Tuple[int, str]]) -> List[Tuple[int, str, List[Reg]]]:
    """[(line, instruction, pending registers it names)] for one kernel."""
    blocks = _blocks(body)
    index = {b[0]: i for i, b in enumerate(blocks) if b[0] is not None}
    succs = []
    for i, (_, _, targets, falls) in enumerate(blocks):
        s = [index[t] for t in targets if t in index]
        if falls and i + 1 < len(blocks):
            s.append(i + 1)
        succs.append(s)
    entry: List[Optional[Queue]] = [None] * len(blocks)
    if blocks:
        entry[0] = ()
    work = [0] if blocks else []
    while work:
        i = work.pop()
        q = entry[i]
        for ins in blocks[i][1]:
            q = _step(q, ins, None)
        for j in succs[i]:
            nq = _join(entry[j], q)
            if nq != entry[j]:
                entry[j] = nq
                work.append(j)
    found = []
    for i, blk in enumerate(blocks):
        q = entry[i]
        if q is None:
            continue
        for ins in blk[1]:
            q = _step(q, ins, lambda ins, regs: found.append((ins.line, ins.text, regs)))
    return found


def kernels(asm: str) -> Dict[str, List[Tuple[int, str]]]:
    """Kernel name -> its (line number, text) lines, from a device assembly file."""
    lines = asm.split("\n")
    out, i = {}, 0
    while i < len(lines):
        m = _FUNC.match(lines[i])
        if not m:
            i += 1
            continue
        j = i + 1
        while j < len(lines) and not lines[j].strip().startswith(".Lfunc_end"):
            j += 1
        out[m.group(1)] = [(k + 1, lines[k]) for k in range(i + 1, j)]
        i = j
    return out


def check_asm(asm: str) -> Dict[str, List[Tuple[int, str, List[Reg]]]]:
    return {name: f for name, body in kernels(asm).items() for f in [check_kernel(body)] if f}


def demangle(name: str) -> str:
    try:
        return subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip() or name
    except OSError:
        return name


if __name__ == "__main__":
    import sys

    bad = 0
    for path in sys.argv[1:]:
        for name, found in check_asm(open(path).read()).items():
            bad += 1
            print(f"{path}: {demangle(name)}: {len(found)} instructions name registers of "
                  f"loads that may be in flight, first: line {found[0][0]} {found[0][1]!r} {found[0][2][:4]}")
    sys.exit(1 if bad else 0)
