"""Wait states after matrix (MFMA) instructions in compiled gfx950 code.

An MFMA writes its result over several passes, and the hardware does not hold
back a later instruction that uses that result: the program must leave enough
independent instructions or `s_nop` wait states in between. This applies to an
MFMA result that a vector ALU instruction reads (`v_accvgpr_read` included)
or writes again, that a memory or LDS store takes as data, or that another MFMA
reads as its A or B operand. A chain of MFMAs that accumulate into the same
registers (srcC = vdst) is resolved by the hardware and is not checked.

REQUIRED holds the wait states for each MFMA shape. The figures are the least
that the compiler itself leaves on straight-line code for that shape:
12 after the 8-pass 16-bit 32x32x16 products and 18 after the 16-pass fp32
32x32x2 product. A shape not listed is held to 20.

`short_paths(asm_text)` parses the assembly that `hipcc -S` writes. It builds
each function's control-flow graph, with blocks split at labels and after
branches, then walks every path backward from each use of an MFMA result to
the MFMA that last wrote it. It reports each use that some path reaches with
too few wait states. The compiler's own count follows the fall-through path
and can miss a shorter path through a taken branch. Each instruction counts
one wait state and `s_nop N` counts N + 1, which never overstates the real
distance.
"""

from __future__ import annotations

import re

REQUIRED = {
    "v_mfma_f32_32x32x16_bf16": 12,
    "v_mfma_f32_32x32x16_f16": 12,
    "v_mfma_f32_32x32x2_f32": 18,
}
UNKNOWN_REQUIRED = 20


def required(opcode: str) -> int:
    return REQUIRED.get(opcode, UNKNOWN_REQUIRED)


_RANGE = re.compile(r"^([va])\[(\d+):(\d+)\]$")
_ONE = re.compile(r"^([va])(\d+)$")


def regs(operand: str) -> set:
    """Vector/accumulation registers an operand names, as ('v', n) / ('a', n)."""
    t = operand.strip().lstrip("-|").rstrip("|")
    m = _RANGE.match(t)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _ONE.match(t)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _split(inst: str):
    parts = inst.split(None, 1)
    ops = parts[1].split(",") if len(parts) > 1 else []
    return parts[0], ops


def _uses(inst: str) -> set:
    """Registers whose pending MFMA result this instruction depends on."""
    op, ops = _split(inst)
    if op.startswith("v_mfma"):
        return set().union(set(), *(regs(o) for o in ops[1:3]))  # A and B only
    if op.startswith("v_"):
        return set().union(set(), *(regs(o) for o in ops))  # reads and the write
    if op.startswith(("ds_write", "buffer_store", "global_store", "flat_store", "scratch_store")):
        return set().union(set(), *(regs(o) for o in ops[1:]))
    return set()


def _wait_states(inst: str) -> int:
    op, ops = _split(inst)
    if op == "s_nop":
        return int(ops[0], 0) + 1
    return 1


def functions(asm: str):
    """(name, instruction/label lines) for each function in the assembly."""
    out, cur, name = [], None, None
    for raw in asm.split("\n"):
        line = raw.split(";")[0].strip()
        if not line:
            continue
        m = re.match(r"^([A-Za-z_][\w.$]*):$", line)
        if m and not line.startswith("."):
            name, cur = m.group(1), []
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            out.append((name, cur))
            cur = None
            continue
        if line.startswith(".LBB") and line.endswith(":"):
            cur.append(line)
        elif not line.startswith("."):
            cur.append(line)
    return out


def _blocks(body):
    blocks = [[None, []]]
    for line in body:
        if line.endswith(":"):
            blocks.append([line[:-1], []])
            continue
        blocks[-1][1].append(line)
        if line.startswith(("s_cbranch", "s_branch")):
            blocks.append([None, []])
    index = {lab: i for i, (lab, _) in enumerate(blocks) if lab}
    preds = {i: [] for i in range(len(blocks))}
    for i, (_, insts) in enumerate(blocks):
        op = insts[-1].split()[0] if insts else ""
        if op.startswith(("s_cbranch", "s_branch")):
            target = insts[-1].split()[1]
            if target in index:
                preds[index[target]].append(i)
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            preds[i + 1].append(i)
    return blocks, preds


def short_paths(asm: str):
    """[(function, instruction, wait states found, wait states required)]
    for every use of an MFMA result that some path reaches too early."""
    need_max = max(max(REQUIRED.values()), UNKNOWN_REQUIRED)
    found = []
    for fname, body in functions(asm):
        blocks, preds = _blocks(body)
        for bi, (_, insts) in enumerate(blocks):
            for ii, inst in enumerate(insts):
                use = _uses(inst)
                if not use:
                    continue
                worst = [None]

                def walk(b, end, dist, pending, seen):
                    j = end - 1
                    insts_b = blocks[b][1]
                    while j >= 0:
                        x = insts_b[j]
                        if x.startswith("v_mfma"):
                            hit = regs(_split(x)[1][0]) & pending
                            if hit:
                                need = required(_split(x)[0])
                                if dist < need and (worst[0] is None or dist - need < worst[0][0] - worst[0][1]):
                                    worst[0] = (dist, need)
                                pending = pending - hit  # older writers of these are covered
                                if not pending:
                                    return
                        dist += _wait_states(x)
                        if dist >= need_max:
                            return
                        j -= 1
                    for p in preds[b]:
                        key = (p, dist, frozenset(pending))
                        if key not in seen:
                            seen.add(key)
                            walk(p, len(blocks[p][1]), dist, pending, seen)

                walk(bi, ii, 0, use, set())
                if worst[0] is not None:
                    found.append((fname, inst, worst[0][0], worst[0][1]))
    return found
