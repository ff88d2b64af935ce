"""Static check of the encoder's device code for one hazard the compiler
cannot see.

The sweep kernel issues its MFMAs from inline asm, so the compiler does not
know their result latency.  If it ever touches an MFMA destination register
itself (say, a register copy between two asm blocks) before the result is
written, it reads a stale value and the scores are silently wrong.  The
epilogue waits explicitly (s_nop) before reading the accumulators; nothing
else may read them early.  This module finds compiler-issued instructions
that touch an MFMA destination within a given number of wait states of the
asm MFMA that writes it, following fall-through and branch targets.
"""
from __future__ import annotations

import re

_VREG = re.compile(r"([va])\[(\d+):(\d+)\]$")
_VONE = re.compile(r"([va])(\d+)$")


def _regs(tok: str) -> set[tuple[str, int]]:
    """Vector registers named by an operand, as (file, index): v and a
    (arch VGPRs and AGPRs) are separate files."""
    m = _VREG.match(tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _VONE.match(tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def kernel_bodies(asm: str, prefix: str) -> dict[str, list[str]]:
    """Device functions whose mangled name starts with prefix -> their lines."""
    start = re.compile(r"^(" + re.escape(prefix) + r"\w*):")
    out, cur = {}, None
    for line in asm.split("\n"):
        m = start.match(line)
        if m:
            cur = out.setdefault(m.group(1), [])
            continue
        if cur is not None:
            cur.append(line)
            if line.strip().startswith("s_endpgm"):
                cur = None
    return out


def early_mfma_reads(body: list[str], limit: int = 20) -> list[tuple[int, str, int]]:
    """(line, instruction, wait states) of compiler instructions that touch an
    asm MFMA's destination fewer than `limit` wait states after its issue."""
    labels = {}
    inasm = []
    flag = False
    for i, raw in enumerate(body):
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            flag = True
        elif t.startswith(";;#ASMEND"):
            flag = False
        inasm.append(flag)
        if t.endswith(":") and not t.startswith(";"):
            labels[t[:-1]] = i
    hits = set()

    def walk(i, pending, budget):
        while i < len(body) and budget > 0 and pending:
            t = body[i].strip()
            if not t or t.startswith((";", ".")) or t.endswith(":"):
                i += 1
                continue
            ops = t.replace(",", " ").split()
            step = int(ops[1]) + 1 if ops[0] == "s_nop" else 1
            if not inasm[i]:
                srcs = set()
                for o in ops[1:]:
                    srcs |= _regs(o)
                for r, d in pending:
                    if r & srcs:
                        hits.add((i + 1, t, d))
            elif ops[0].startswith("v_mfma"):
                return
            pending = [(r, d + step) for r, d in pending if d + step < limit]
            budget -= 1
            if ops[0] == "s_branch":
                i = labels.get(ops[1], len(body))
                continue
            if ops[0].startswith("s_cbranch") and ops[1] in labels:
                walk(labels[ops[1]], pending, budget)
            if ops[0] == "s_endpgm":
                return
            i += 1

    for i, raw in enumerate(body):
        t = raw.strip()
        if inasm[i] and t.startswith("v_mfma"):
            walk(i + 1, [(_regs(t.replace(",", " ").split()[1]), 0)], 60)
    return sorted(hits)
