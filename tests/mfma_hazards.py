"""Static check of MFMA result hazards in the gfx950 assembly of this library.

A matrix instruction (v_mfma_*) writes its destination registers several
cycles after it issues; an instruction that reads those registers before
then gets the old values.  The compiler pads such reads with wait states
(s_nop) in straight-line code, but it can miss a path that leaves the block
through a branch.  This checker parses the assembly hipcc writes for one
source file, builds each kernel's control-flow graph, and for every MFMA
walks every path forward, counting wait states (one per instruction,
s_nop n counts n + 1), until the destination is read, rewritten, or enough
wait states have passed.  An MFMA that takes the destination as its
accumulator input is not counted as a reader (the hardware forwards an
accumulator from one MFMA to the next); its A and B operands are.

The required count is taken from the compiler itself.  A probe kernel per
MFMA opcode (``probe_source``) reads the result right after the instruction,
so the compiler pads that read with exactly the wait states its hazard rule
asks for (``probed_requirements``).  Without a probe, the fallback is the
smallest number of wait states the compiler leaves between an MFMA and a read
of its result inside one basic block of the checked code, which can only
overstate the rule.  Every path must leave at least the required count.
"""

from __future__ import annotations

import os
import re
import subprocess
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Set, Tuple

REG_RE = re.compile(r"\b([vas])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
BRANCH_RE = re.compile(r"^s_(c?branch\w*)\s+(\S+)")


@dataclass
class Instr:
    op: str
    text: str
    dst: Set[str] = field(default_factory=set)
    src: Set[str] = field(default_factory=set)
    srcc: Set[str] = field(default_factory=set)  # MFMA accumulator input
    waits: int = 1


def _regs(operand: str) -> Set[str]:
    out = set()
    for m in REG_RE.finditer(operand):
        kind = m.group(1)
        if kind == "s":
            continue
        if m.group(4) is not None:
            out.add(f"{kind}{m.group(4)}")
        else:
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add(f"{kind}{r}")
    return out


# instructions whose first register operand is read, not written
_STORE_PREFIXES = ("ds_write", "ds_store", "global_store", "buffer_store", "flat_store",
                   "scratch_store", "global_atomic", "ds_add", "ds_max", "ds_min")


def parse_instr(line: str) -> Optional[Instr]:
    line = line.split(";")[0].strip()
    if not line or line.endswith(":") or line.startswith("."):
        return None
    parts = line.split(None, 1)
    op = parts[0]
    args = parts[1] if len(parts) > 1 else ""
    ins = Instr(op=op, text=line)
    if op == "s_nop":
        ins.waits = int(args.strip(), 0) + 1
        return ins
    operands = [a.strip() for a in args.split(",")] if args else []
    if not operands:
        return ins
    if op.startswith(_STORE_PREFIXES) or op.startswith("s_"):
        for o in operands:
            ins.src |= _regs(o)
        return ins
    ins.dst = _regs(operands[0])
    if op.startswith("v_mfma") and len(operands) >= 4:
        for o in operands[1:3]:
            ins.src |= _regs(o)
        ins.srcc = _regs(operands[3])
        return ins
    for o in operands[1:]:
        ins.src |= _regs(o)
    return ins


@dataclass
class Kernel:
    name: str
    instrs: List[Instr]
    labels: Dict[str, int]


def parse_kernels(asm: str) -> List[Kernel]:
    kernels = []
    cur = None
    for raw in asm.splitlines():
        line = raw.split(";")[0].rstrip()
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = Kernel(m.group(1), [], {})
            kernels.append(cur)
            continue
        if cur is None:
            continue
        lm = re.match(r"^(\.L\w+):", line.strip())
        if lm:
            cur.labels[lm.group(1)] = len(cur.instrs)
            continue
        if line.strip().startswith(".Lfunc_end"):
            cur = None
            continue
        ins = parse_instr(line)
        if ins is not None:
            cur.instrs.append(ins)
    return kernels


def successors(k: Kernel, i: int) -> List[int]:
    ins = k.instrs[i]
    if ins.op == "s_endpgm":
        return []
    m = BRANCH_RE.match(ins.text)
    if m:
        target = k.labels.get(m.group(2))
        nxt = [] if ins.op == "s_branch" else [i + 1]
        if target is not None:
            nxt.append(target)
        return [j for j in nxt if j < len(k.instrs)]
    return [i + 1] if i + 1 < len(k.instrs) else []


def _is_mfma(ins: Instr) -> bool:
    return ins.op.startswith("v_mfma")


def min_distance_to_read(k: Kernel, i: int, limit: int) -> Optional[Tuple[int, int]]:
    """Fewest wait states on any path from MFMA i to an instruction reading
    its destination (None if every path rewrites it or passes `limit`)."""
    dst = k.instrs[i].dst
    best: Optional[Tuple[int, int]] = None
    # (position, wait states so far); visit each position with its smallest count
    seen: Dict[int, int] = {}
    stack = [(j, 0) for j in successors(k, i)]
    while stack:
        j, w = stack.pop()
        if w >= limit or (j in seen and seen[j] <= w):
            continue
        seen[j] = w
        ins = k.instrs[j]
        if _is_mfma(ins) and ins.dst == dst:
            continue  # accumulation chain (forwarded) or a full rewrite
        if ins.src & dst:
            if best is None or w < best[0]:
                best = (w, j)
            continue
        if dst <= ins.dst:
            continue  # rewritten before any read
        for s in successors(k, j):
            stack.append((s, w + ins.waits))
    return best


def same_block_distances(k: Kernel) -> List[Tuple[str, int]]:
    """(MFMA opcode, wait states) the compiler left between an MFMA and a read
    of its result within one basic block (no label or branch in between)."""
    label_pos = set(k.labels.values())
    out = []
    for i, ins in enumerate(k.instrs):
        if not _is_mfma(ins):
            continue
        w = 0
        for j in range(i + 1, len(k.instrs)):
            if j in label_pos:
                break
            nj = k.instrs[j]
            if _is_mfma(nj) and nj.dst == ins.dst:
                break
            if nj.src & ins.dst:
                out.append((ins.op, w))
                break
            if ins.dst <= nj.dst or BRANCH_RE.match(nj.text) or nj.op == "s_endpgm":
                break
            w += nj.waits
    return out


def required_waits(kernels: List[Kernel]) -> Dict[str, int]:
    """Per MFMA opcode, the fewest wait states the compiler leaves before a
    read of its result in straight-line code: its own hazard rule."""
    req: Dict[str, int] = {}
    for k in kernels:
        for op, w in same_block_distances(k):
            req[op] = min(req.get(op, w), w)
    return req


def check(asm: str, required: Optional[Dict[str, int]] = None):
    """Violations [(kernel, mfma text, wait states, reader text, required)] and
    the per-opcode requirements used (an opcode never read in straight-line
    code is held to the largest requirement seen)."""
    kernels = parse_kernels(asm)
    if required is None:
        required = required_waits(kernels)
    fallback = max(required.values()) if required else 0
    bad = []
    for k in kernels:
        for i, ins in enumerate(k.instrs):
            if not _is_mfma(ins):
                continue
            need = required.get(ins.op, fallback)
            r = min_distance_to_read(k, i, need)
            if r is not None and r[0] < need:
                bad.append((k.name, ins.text, r[0], k.instrs[r[1]].text, need))
    return bad, required


def device_asm(src: str, flags: List[str], hipcc: str) -> str:
    """gfx950 assembly of one HIP source, built with the library's flags."""
    cmd = [hipcc, *[f for f in flags if f != "-fPIC"], "--cuda-device-only", "-S", src, "-o", "-"]
    return subprocess.run(cmd, check=True, capture_output=True, text=True).stdout


# One probe kernel per MFMA opcode the library uses: operand type and builtin.
PROBES = {
    "v_mfma_f32_16x16x32_bf16": ("bf16x8", "__builtin_amdgcn_mfma_f32_16x16x32_bf16"),
    "v_mfma_f32_16x16x16_bf16": ("s16x4", "__builtin_amdgcn_mfma_f32_16x16x16bf16_1k"),
    "v_mfma_f32_16x16x4_f32": ("float", "__builtin_amdgcn_mfma_f32_16x16x4f32"),
}


def probe_source() -> str:
    """A HIP source with one kernel per probed opcode whose result is read by
    the next instruction."""
    lines = [
        "#include <hip/hip_runtime.h>",
        "typedef __attribute__((ext_vector_type(4))) float f32x4;",
        "typedef __attribute__((ext_vector_type(4))) short s16x4;",
        "typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;",
    ]
    for n, (ty, builtin) in enumerate(PROBES.values()):
        lines += [
            f"__global__ void probe{n}(const {ty}* a, const {ty}* b, float* o) {{",
            "  f32x4 c = {0.f, 0.f, 0.f, 0.f};",
            f"  c = {builtin}(a[threadIdx.x], b[threadIdx.x], c, 0, 0, 0);",
            "  o[threadIdx.x] = c[0] + 1.0f;",
            "}",
        ]
    return "\n".join(lines) + "\n"


def probed_requirements(flags: List[str], hipcc: str, workdir: str) -> Dict[str, int]:
    """Wait states the compiler leaves before reading each probed MFMA's
    result in straight-line code."""
    src = os.path.join(workdir, "mfma_probe.hip")
    with open(src, "w") as f:
        f.write(probe_source())
    req: Dict[str, int] = {}
    for k in parse_kernels(device_asm(src, flags, hipcc)):
        for op, w in same_block_distances(k):
            req[op] = min(req.get(op, w), w)
    return req

