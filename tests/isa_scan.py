"""Checks on the gfx950 assembly of this library's own kernels.

mfma_srcc_gaps: for every MFMA that reads an accumulator input (SrcC) from
registers, the first later non-MFMA instruction that writes one of those
registers, when it comes fewer than `limit` wait states after the MFMA (an
instruction is one wait state, s_nop N is N + 1).  Such writes were measured
to corrupt the MFMA's result on gfx950 even where the compiler's hazard model
allowed them, so the kernels fence their MFMA groups and this scan keeps it so.

forbidden: scalar-cache stores, atomics and cache write-back/discard, and
packed fp32 VALU instructions, none of which the kernels may contain.
"""
from __future__ import annotations

import re

_KERNEL = re.compile(r"^(_Z\S+):")


def _regs(tok: str) -> set[tuple[str, int]]:
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _instructions(text: str):
    """(line number, kernel, instruction text) for every instruction line."""
    kernel = "?"
    for no, line in enumerate(text.splitlines(), 1):
        m = _KERNEL.match(line)
        if m:
            kernel = m.group(1)
            continue
        t = line.split(";", 1)[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        yield no, kernel, t


def _writes(inst: str) -> set[tuple[str, int]]:
    op, _, rest = inst.partition(" ")
    if not rest:
        return set()
    if op.startswith(("v_cmp", "v_cmpx", "ds_write", "ds_store", "global_store", "buffer_store",
                      "global_atomic", "buffer_atomic", "global_load_lds", "buffer_load_lds")):
        return set()
    if op.startswith("buffer_load") and rest.split()[-1] == "lds":
        return set()  # direct-to-LDS form: the first operand is the offset it reads
    if op.startswith(("v_", "ds_", "global_load", "buffer_load", "flat_load", "scratch_load")):
        return _regs(rest.split(",")[0])
    return set()


def mfma_srcc_gaps(text: str, limit: int = 8):
    insts = list(_instructions(text))
    hits = []
    for i, (no, kernel, inst) in enumerate(insts):
        if not inst.startswith("v_mfma"):
            continue
        ops = inst.split(None, 1)[1].split(",")
        srcc = _regs(ops[3]) if len(ops) > 3 else set()
        if not srcc:
            continue
        ws = 0
        for no2, kernel2, inst2 in insts[i + 1:]:
            if kernel2 != kernel or ws >= limit:
                break
            if inst2.startswith("s_nop"):
                ws += int(inst2.split()[1], 0) + 1
                continue
            if not inst2.startswith("v_mfma") and _writes(inst2) & srcc:
                hits.append((kernel, no, inst, no2, inst2, ws))
                break
            ws += 1
    return hits


_FORBIDDEN = re.compile(r"^\s*(s_store|s_buffer_store|s_scratch_store|s_atomic|s_buffer_atomic|"
                        r"s_dcache_wb|s_dcache_discard|v_pk_add_f32|v_pk_mul_f32|v_pk_fma_f32)")


def forbidden(text: str):
    return [(no, line.strip()) for no, line in enumerate(text.splitlines(), 1) if _FORBIDDEN.match(line)]
