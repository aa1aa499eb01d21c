"""Static check of compiled gfx950 assembly: no instruction may read or write
the destination VGPRs of a vector-memory load that has not been retired by a
preceding s_waitcnt vmcnt.

Kernels that issue their global loads through inline asm (so that the
compiler's own wait insertion does not serialise a prefetch ring) take on the
compiler's job of keeping those registers untouched until the data lands; a
load whose result is never consumed is the typical way to break it, since the
compiler then hands its registers to another value. The walk is linear over
the function body (branches are ignored, so both sides of an if/else apply
their waits); every global_load* counts as one vmcnt event, in issue order.
A load whose destination overlaps a pending load's is not a violation: loads
return in issue order, so the later one's data lands last (the two sides of
an if/else that load the same registers look like this to a linear walk);
its address operands are checked like any other read.
"""
import re


def _regs(text):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def violations(body_lines):
    """List of (line, instruction, load_line) for touches of pending loads."""
    pending = []          # (line, dest VGPRs or None for LDS-DMA loads), issue order
    found = []
    for k, line in enumerate(body_lines):
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        op = t.split()[0]
        if op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", t)
            if m:
                n = int(m.group(1))
                pending = pending[len(pending) - n:] if 0 < n < len(pending) else (
                    [] if n == 0 else pending)
            continue
        is_load = op.startswith("global_load") or op.startswith("buffer_load")
        operands = t[len(op):]
        if is_load and "lds" not in op and "," in operands:
            operands = operands.split(",", 1)[1]   # the destination is a write
        touched = _regs(operands)
        for pk, dest in pending:
            if dest and touched & dest:
                found.append((k, t, pk))
                break
        if is_load:
            dst = None if "lds" in op else _regs(t[len(op):].split(",")[0])
            pending.append((k, dst))
    return found


def check_asm(text, symbol_regex):
    """{kernel symbol: violations} for every function matching the regex."""
    out = {}
    for m in re.finditer(r"^(%s):" % symbol_regex, text, re.M):
        start = m.end()
        end = text.index(".Lfunc_end", start)
        out[m.group(1)] = violations(text[start:end].splitlines())
    return out
