"""Check gfx950 device assembly for MFMA results read too early.

hipcc leaves a number of wait states between an MFMA and the first non-MFMA
instruction that reads or overwrites its destination registers (gfx950 does
not interlock those dependencies).  On straight-line code it always leaves
at least the count in ``WAIT_STATES`` for that MFMA opcode (8 after a
16x16x32 product, 12 after a 32x32x16 one, read off hipcc's own output);
across a conditional branch that skips a block it has been seen to leave
only one, so the consumer read the accumulator's old value and the kernel
returned wrong, run-to-run different results.  This module walks every
control-flow path after each MFMA (fall-through and branch targets) and
reports any read (RAW) or non-MFMA write (WAW) of its destination that
comes sooner.  An MFMA opcode missing from the table is reported as well,
so that a new product shape cannot pass unchecked.

    python -m block_causal_transformer_amd.hazard_check FILE.s [...]

``build`` runs it on the assembly of every HIP source and fails on a hit.
"""
from __future__ import annotations

import re
import sys

# Wait states hipcc leaves between each MFMA and a VALU access of its result.
WAIT_STATES = {
    "v_mfma_f32_16x16x32_bf16": 8,
    "v_mfma_f32_16x16x32_f16": 8,
    "v_mfma_f32_32x32x16_bf16": 12,
    "v_mfma_f32_32x32x16_f16": 12,
}
MIN_STATES = 8  # the smallest entry (kept for callers that pass a fixed count)

_STORES = ("ds_write", "global_store", "buffer_store", "scratch_store", "flat_store")


def _regs(tok: str) -> set:
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _parse(lines):
    ins, labels = [], {}
    for ln in lines:
        s = ln.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            labels[s[:-1]] = len(ins)
            continue
        if s.startswith("."):
            continue
        parts = s.split(None, 1)
        args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        ins.append((parts[0], args, s))
    return ins, labels


def _kernels(text: str):
    """(name, lines) of every function body in an assembly file: from the
    function's label to its end marker (.Lfunc_endN), so that code after an
    early s_endpgm (a returning path) is checked too."""
    out, name, cur = [], None, []
    for ln in text.split("\n"):
        m = re.match(r"^([A-Za-z_][\w.$]*):", ln)
        if m and not ln.startswith(".") and name is None and not m.group(1).startswith(".L"):
            name, cur = m.group(1), []
            continue
        if name is not None:
            if re.match(r"^\.Lfunc_end\d+:", ln):
                out.append((name, cur))
                name = None
                continue
            cur.append(ln)
    if name is not None:
        out.append((name, cur))
    return out


def check_function(lines, min_states=None):
    """List of (mfma text, consumer text, wait states) violations.  The
    required count is the opcode's entry in WAIT_STATES, or ``min_states``
    when given; an unknown MFMA opcode is itself a violation (wait states -1)."""
    ins, labels = _parse(lines)
    bad = []
    for i, (op, args, text) in enumerate(ins):
        if not op.startswith("v_mfma") or not args:
            continue
        need = min_states if min_states is not None else WAIT_STATES.get(op.split("_e64")[0])
        if need is None:
            bad.append((text, "unknown MFMA opcode %s" % op, -1))
            continue
        dst = _regs(args[0])
        stack, seen = [(i + 1, 0)], set()
        while stack:
            j, st = stack.pop()
            if st >= need or j >= len(ins) or (j, st) in seen:
                continue
            seen.add((j, st))
            op2, a2, text2 = ins[j]
            if op2.startswith("v_mfma"):
                # another MFMA may take the result as an operand (the
                # hardware forwards it); one that overwrites it ends the hazard
                if a2 and _regs(a2[0]) & dst:
                    continue
            else:
                is_store = op2.startswith(_STORES)
                srcs = a2 if is_store else a2[1:]
                used = set()
                for a in srcs:
                    used |= _regs(a)
                # RAW: a source reads the result; WAW: the destination
                # (the first operand of every non-store) overwrites it
                if used & dst or (not is_store and a2 and _regs(a2[0]) & dst):
                    bad.append((text, text2, st))
            nst = st + (int(a2[0], 0) + 1 if op2 == "s_nop" else 1)
            if op2 == "s_endpgm":
                continue
            if op2 == "s_branch" or op2.startswith("s_cbranch"):
                if a2[0] not in labels:
                    raise ValueError("branch to %s, which is not in the function" % a2[0])
                stack.append((labels[a2[0]], nst))
                if op2 == "s_branch":
                    continue
            stack.append((j + 1, nst))
    return bad


def check_text(text: str, min_states=None):
    """{kernel: violations} for every kernel with at least one."""
    res = {}
    for name, lines in _kernels(text):
        bad = check_function(lines, min_states)
        if bad:
            res[name] = bad
    return res


def check_file(path: str, min_states=None):
    with open(path) as f:
        return check_text(f.read(), min_states)


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    status = 0
    for path in argv:
        res = check_file(path)
        for name, bad in res.items():
            status = 1
            print("%s: %s: %d MFMA result access(es) too early (or unknown MFMA)" % (path, name, len(bad)))
            for mf, use, st in bad[:5]:
                print("    %s  ->  %s  (after %d)" % (mf, use, st))
    return status


if __name__ == "__main__":
    sys.exit(main())
