"""Static check of the gfx950 assembly of libkda for one MFMA hazard pattern.

An MFMA writes its accumulator registers several cycles after issue; a later
instruction that reads them needs enough independent instructions (wait states)
in between.  The compiler inserts s_nop for straight-line code, but a read
reached through a branch that skips code (e.g. `s_cbranch_execz` over a loop)
has been seen with only a few instructions after the MFMA on that path, reading a
stale accumulator element.  This check flags every MFMA-result read that is
reachable from the MFMA through a forward branch with fewer than `min_wait` wait
states on that path (straight-line sequences, where the compiler places its own
s_nop, are not flagged).

Usage: python -m kda_gated_delta_rule_amd.isa_lint  (compiles the sources with
hipcc -S for gfx950 and prints the findings; exit status 1 if any).
"""
import os
import re
import subprocess
import sys
import tempfile

from . import _build

_REG = re.compile(r"\b([av])\[(\d+):(\d+)\]|\b([av])(\d+)\b")
_MFMA = re.compile(r"^\s*v_mfma\w*\s+(\S+?),\s*(.*)$")
_LABEL = re.compile(r"^(\.?LBB\w+|\w+):")
_BRANCH = re.compile(r"^\s*s_cbranch_\w+\s+(\S+)|^\s*s_branch\s+(\S+)")
_NOP = re.compile(r"^\s*s_nop\s+(\d+)")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _split_operands(line):
    body = line.split(";")[0].strip()
    parts = body.split(None, 1)
    if len(parts) < 2:
        return parts[0] if parts else "", "", ""
    ops = parts[1].split(",", 1)
    return parts[0], ops[0], ops[1] if len(ops) > 1 else ""


def functions(asm_text):
    """Yields (name, [lines]) for each kernel in a device assembly file."""
    name, lines = None, []
    for ln in asm_text.splitlines():
        m = re.match(r"^(_Z\w+):", ln)
        if m:
            if name:
                yield name, lines
            name, lines = m.group(1), []
        elif name is not None:
            lines.append(ln)
            if ln.strip() == "s_endpgm":
                yield name, lines
                name, lines = None, []


def check_function(lines, min_wait=10):
    insts = []  # (kind, text, label)
    for ln in lines:
        s = ln.strip()
        if not s or s.startswith(";") or s.startswith("."):
            m = _LABEL.match(s)
            if m and s.startswith(".LBB"):
                insts.append(("label", s, m.group(1)))
            continue
        m = _LABEL.match(s)
        if m:
            insts.append(("label", s, m.group(1)))
            continue
        insts.append(("inst", s, None))
    label_pos = {lab: i for i, (k, _, lab) in enumerate(insts) if k == "label"}

    def ws(i):
        k, s, _ = insts[i]
        if k != "inst":
            return 0
        m = _NOP.match(s)
        return int(m.group(1)) + 1 if m else 1

    findings = []
    for m_i, (k, s, _) in enumerate(insts):
        if k != "inst":
            continue
        mm = _MFMA.match(s)
        if not mm:
            continue
        dst = _regs(mm.group(1))
        for r_i in range(m_i + 1, len(insts)):
            k2, s2, _ = insts[r_i]
            if k2 != "inst":
                continue
            op, first, rest = _split_operands(s2)
            if op.startswith("v_mfma"):
                d2 = _regs(first)
                srcs = _regs(rest)
                if d2 == dst:  # chained accumulation into the same registers
                    break
                if dst & srcs:
                    break
                continue
            if op.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
                continue
            reads = _regs(rest) | (_regs(first) if op.startswith(("ds_write", "global_store",
                                                                   "buffer_store", "flat_store",
                                                                   "scratch_store")) else set())
            if op.startswith("v_accvgpr_read"):
                reads = _regs(rest)
            if dst & reads:
                # shortest path from the MFMA to this read through a forward branch
                best = None
                for b_i in range(m_i + 1, r_i):
                    kb, sb, _ = insts[b_i]
                    bm = _BRANCH.match(sb) if kb == "inst" else None
                    if not bm:
                        continue
                    tgt = bm.group(1) or bm.group(2)
                    l_i = label_pos.get(tgt)
                    if l_i is None or not (b_i < l_i <= r_i):
                        continue
                    path = sum(ws(i) for i in range(m_i + 1, b_i + 1)) + sum(ws(i) for i in range(l_i, r_i))
                    best = path if best is None else min(best, path)
                if best is not None and best < min_wait:
                    findings.append((m_i, r_i, best, s, s2))
                break
            if dst & _regs(first) and not op.startswith(("ds_", "global_", "buffer_", "s_")):
                break  # overwritten before any read
    return findings


def device_asm(sources=None):
    """Compiles the HIP sources to gfx950 assembly (device only); returns the text."""
    sources = sources or [s for s in _build.sources() if s.endswith(".hip")]
    out = []
    with tempfile.TemporaryDirectory() as d:
        for src in sources:
            dst = os.path.join(d, os.path.basename(src) + ".s")
            flags = [f for f in _build.FLAGS if f not in ("-shared", "-fPIC")]
            cmd = ["hipcc"] + flags + ["-I" + _build.INCLUDE, "-I" + _build.CSRC,
                                       "--cuda-device-only", "-S", src, "-o", dst]
            subprocess.run(cmd, check=True, capture_output=True)
            out.append(open(dst).read())
    return "\n".join(out)


def lint(asm_text=None, min_wait=10):
    asm_text = asm_text if asm_text is not None else device_asm()
    found = []
    for name, lines in functions(asm_text):
        for f in check_function(lines, min_wait):
            found.append((name,) + f)
    return found


if __name__ == "__main__":
    res = lint()
    for name, m_i, r_i, best, s, s2 in res:
        print("%s: MFMA '%s' -> read '%s' with %d wait states on a branch path"
              % (name[:90], s, s2, best))
    print("%d finding(s)" % len(res))
    sys.exit(1 if res else 0)
