"""Static checks of the attention kernels' gfx950 assembly.

The P V products of the forward kernel are inline-asm MFMAs on AGPR
accumulators. The compiler's hazard recognizer does not look inside inline
asm, so two orders are the kernel's own responsibility:

* an MFMA result read or overwritten by any other instruction: at least
  ``MFMA_RESULT_WAIT`` wait states after the MFMA (16-pass XDL op + 2);
* a VGPR written by a VALU instruction and read by an inline-asm MFMA as its
  A or B operand: at least ``VALU_TO_MFMA_WAIT`` wait states in between.

A wait state is one issued instruction, or N + 1 for ``s_nop N``. The scan
walks the control-flow graph of each kernel (fall-through and branch edges)
from every inline-asm MFMA, forward for the first rule and backward for the
second. It also reports the scratch (spill) size of each kernel from the
assembler metadata: spill code around the inline asm would move accumulators
behind the kernel's back.

A third check looks at the innermost loops that hold the kernels' MFMAs (the
per-block loops). The kernels fill LDS with LDS-DMA written as inline asm,
which the compiler does not count, so any vector-memory wait the compiler puts
inside such a loop (for a spill reload, or for a load issued before the loop)
also waits for the DMA of the next block in flight. Those loops must hold no
scratch access and no compiler-placed vmcnt wait; the kernels' own waits are
inline asm.
"""

from __future__ import annotations

import re
from dataclasses import dataclass, field

MFMA_RESULT_WAIT = 18
VALU_TO_MFMA_WAIT = 2

_RANGE = re.compile(r"\b([av])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"\b([av])(\d+)\b")


def regs(text: str) -> set[tuple[str, int]]:
    """The a/v registers an operand string names."""
    out: set[tuple[str, int]] = set()
    for kind, lo, hi in _RANGE.findall(text):
        out.update((kind, r) for r in range(int(lo), int(hi) + 1))
    stripped = _RANGE.sub(" ", text)
    for kind, r in _SINGLE.findall(stripped):
        out.add((kind, int(r)))
    return out


@dataclass
class Instr:
    op: str
    operands: str
    asm: bool  # written by inline asm
    label_before: list[str] = field(default_factory=list)

    @property
    def waits(self) -> int:
        if self.op == "s_nop":
            return int(self.operands.strip(), 0) + 1
        return 1

    def operand_list(self) -> list[str]:
        return [o.strip() for o in self.operands.split(",")] if self.operands.strip() else []


@dataclass
class Kernel:
    name: str
    instrs: list[Instr]
    labels: dict[str, int]
    scratch: int | None = None
    vgpr_spills: int | None = None


def parse(asm_text: str, name_filter: str = "sta_attention_kernel") -> list[Kernel]:
    kernels: list[Kernel] = []
    cur: Kernel | None = None
    in_asm = False
    pending: list[str] = []
    meta_kernel = None
    scratch_of: dict[str, int] = {}
    spills_of: dict[str, int] = {}
    for raw in asm_text.splitlines():
        s = raw.strip()
        if s.startswith(".name:"):
            meta_kernel = s.split(":", 1)[1].strip()
        if s.startswith(".private_segment_fixed_size:") and meta_kernel is not None:
            scratch_of[meta_kernel] = int(s.split(":", 1)[1])
        if s.startswith(".vgpr_spill_count:") and meta_kernel is not None:
            spills_of[meta_kernel] = int(s.split(":", 1)[1])
        m = re.match(r"^(\S+):\s*(;.*)?$", raw)
        if m and not raw.startswith((" ", "\t")):
            label = m.group(1)
            if name_filter in label and not label.startswith("."):
                cur = Kernel(label, [], {})
                kernels.append(cur)
                pending = []
                continue
            if cur is not None:
                if label.startswith(".Lfunc_end"):
                    cur = None
                    continue
                pending.append(label)
            continue
        if cur is None:
            continue
        if "#ASMSTART" in s:
            in_asm = True
            continue
        if "#ASMEND" in s:
            in_asm = False
            continue
        body = raw.split(";")[0].strip()
        if not body or body.startswith("."):
            continue
        parts = body.split(None, 1)
        ins = Instr(parts[0], parts[1] if len(parts) > 1 else "", in_asm, pending)
        for lb in pending:
            cur.labels[lb] = len(cur.instrs)
        pending = []
        cur.instrs.append(ins)
    for k in kernels:
        k.scratch = scratch_of.get(k.name)
        k.vgpr_spills = spills_of.get(k.name)
    return kernels


def _branch_target(ins: Instr) -> str | None:
    if ins.op.startswith("s_cbranch") or ins.op == "s_branch":
        return ins.operands.strip()
    return None


def successors(k: Kernel, i: int) -> list[int]:
    ins = k.instrs[i]
    out = []
    tgt = _branch_target(ins)
    if tgt is not None:
        out.append(k.labels[tgt])
    if ins.op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(k.instrs):
        out.append(i + 1)
    return out


def predecessors_map(k: Kernel) -> list[list[int]]:
    preds: list[list[int]] = [[] for _ in k.instrs]
    for i in range(len(k.instrs)):
        for j in successors(k, i):
            preds[j].append(i)
    return preds


def is_asm_mfma(ins: Instr) -> bool:
    return ins.asm and ins.op.startswith("v_mfma")


def check_result_reads(k: Kernel) -> list[str]:
    """Non-MFMA instructions touching an inline-asm MFMA's destination too early."""
    problems = []
    for i, ins in enumerate(k.instrs):
        if not is_asm_mfma(ins):
            continue
        dst = regs(ins.operand_list()[0])
        # (position, wait states already elapsed)
        stack = [(j, 0) for j in successors(k, i)]
        seen: dict[int, int] = {}
        while stack:
            j, w = stack.pop()
            if w >= MFMA_RESULT_WAIT:
                continue
            if seen.get(j, -1) >= MFMA_RESULT_WAIT - w:
                continue
            seen[j] = MFMA_RESULT_WAIT - w
            nxt = k.instrs[j]
            chained = is_asm_mfma(nxt) and regs(nxt.operand_list()[0]) == dst and regs(nxt.operand_list()[3]) == dst
            if not chained and not (is_asm_mfma(nxt) and not (regs(nxt.operands) & dst)):
                if regs(nxt.operands) & dst:
                    problems.append(f"{k.name}: {nxt.op} {nxt.operands} at #{j}, {w} wait states after "
                                    f"asm MFMA #{i} writing {ins.operand_list()[0]}")
                    continue
            stack.extend((s, w + nxt.waits) for s in successors(k, j))
    return problems


def check_operand_writes(k: Kernel) -> list[str]:
    """VALU writes of an inline-asm MFMA's A/B operands too close before it."""
    problems = []
    preds = predecessors_map(k)
    for i, ins in enumerate(k.instrs):
        if not is_asm_mfma(ins):
            continue
        ops = ins.operand_list()
        src = regs(ops[1]) | regs(ops[2])
        stack = [(p, 0) for p in preds[i]]
        seen: set[tuple[int, int]] = set()
        while stack:
            j, w = stack.pop()
            if w >= VALU_TO_MFMA_WAIT or (j, w) in seen:
                continue
            seen.add((j, w))
            prev = k.instrs[j]
            if prev.op.startswith("v_") and not prev.op.startswith("v_mfma"):
                dst = prev.operand_list()[0] if prev.operand_list() else ""
                if regs(dst) & src:
                    problems.append(f"{k.name}: {prev.op} {prev.operands} at #{j} writes an operand of "
                                    f"asm MFMA #{i} after {w} wait states")
                    continue
            stack.extend((p, w + prev.waits) for p in preds[j])
    return problems


def innermost_loops(k: Kernel) -> list[tuple[int, int]]:
    """(first, last) instruction index of each innermost loop: a header and its
    furthest back edge, holding no other loop."""
    last_of: dict[int, int] = {}
    for i, ins in enumerate(k.instrs):
        tgt = _branch_target(ins)
        if tgt is not None and k.labels[tgt] <= i:
            h = k.labels[tgt]
            last_of[h] = max(last_of.get(h, i), i)
    regions = sorted(last_of.items())
    out = []
    for h, e in regions:
        if not any((h2, e2) != (h, e) and h <= h2 and e2 <= e for h2, e2 in regions):
            out.append((h, e))
    return out


def check_block_loops(k: Kernel, min_mfma: int = 32) -> list[str]:
    """Scratch accesses and compiler-placed vmcnt waits inside the innermost
    loops with at least `min_mfma` MFMAs."""
    problems = []
    for h, e in innermost_loops(k):
        body = k.instrs[h:e + 1]
        if sum(ins.op.startswith("v_mfma") for ins in body) < min_mfma:
            continue
        for j, ins in enumerate(body):
            if ins.op.startswith("scratch_"):
                problems.append(f"{k.name}: {ins.op} {ins.operands} at #{h + j} inside the block loop #{h}-#{e}")
            if ins.op == "s_waitcnt" and "vmcnt" in ins.operands and not ins.asm:
                problems.append(f"{k.name}: compiler wait {ins.operands} at #{h + j} inside the block loop #{h}-#{e}")
    return problems
