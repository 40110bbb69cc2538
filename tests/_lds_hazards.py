"""Dataflow check on gfx950 assembly: no compiler-generated instruction may touch a
register that an inline-asm LDS read (ds_read_*) is still filling.

The kernels issue some LDS reads from inline asm and wait for them with an
explicit s_waitcnt lgkmcnt(N); the compiler sees the destination as written
at the asm statement. A copy, spill or use it placed between the read and its
wait would see data that has not arrived. The check walks the control-flow
graph of each kernel, keeping per block the reads that may still be in flight
(aligned by issue order, so that lgkmcnt(N) retires all but the N most recent),
and reports every compiler instruction that names one of their registers.
"""
import re

REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
LABEL = re.compile(r"^(\.?[A-Za-z_$][\w.$]*):")


def vregs(s):
    out = set()
    for m in REG.finditer(s):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return frozenset(out)


def parse(body):
    """Basic blocks of a kernel body: list of (label, [(kind, op, text, lineno)]),
    kind 'asm' for inline-asm lines, 'cc' for compiler instructions."""
    blocks = [[None, []]]
    in_asm = False
    for ln, raw in enumerate(body.split("\n")):
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True; continue
        if t.startswith(";;#ASMEND"):
            in_asm = False; continue
        code = t.split(";")[0].strip()
        if not code:
            continue
        m = LABEL.match(code)
        if m and not in_asm:
            blocks.append([m.group(1), []])
            continue
        if code.startswith("."):
            continue
        op = code.split()[0]
        blocks[-1][1].append(("asm" if in_asm else "cc", op, code, ln))
        if not in_asm and (op.startswith("s_branch") or op.startswith("s_cbranch") or op == "s_endpgm"):
            blocks.append([None, []])
    return [b for b in blocks if b[1] or b[0]]


def merge(a, b):
    """Join of two in-flight lists, aligned from the most recent read."""
    n = max(len(a), len(b))
    out = []
    for i in range(n, 0, -1):
        x = a[-i] if i <= len(a) else frozenset()
        y = b[-i] if i <= len(b) else frozenset()
        out.append(x | y)
    return tuple(out)


def transfer(state, insts, bad=None):
    """In-flight list after a block; appends violations to bad if given."""
    pend = list(state)
    for kind, op, code, ln in insts:
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", code)
            if m:
                n = int(m.group(1))
                pend = pend[len(pend) - n:] if n < len(pend) else pend
            continue
        if kind == "asm":
            if op.startswith("ds_read"):
                pend.append(vregs(code.split(None, 1)[1].split(",")[0]))
            continue
        if bad is not None and " " in code:
            touched = vregs(code.split(None, 1)[1])
            if any(p & touched for p in pend):
                bad.append((ln, code))
        if op.startswith("ds_") or op.startswith("s_load") or op.startswith("s_buffer_load"):
            pend.append(frozenset())
        if op == "s_endpgm":
            pend = []
    return tuple(pend[-64:])


def check_kernel(body):
    """(line, instruction) of every compiler instruction that touches a register
    of an inline-asm LDS read that may still be in flight."""
    blocks = parse(body)
    index = {b[0]: i for i, b in enumerate(blocks) if b[0]}
    succ = []
    for i, (lab, insts) in enumerate(blocks):
        s = []
        last = insts[-1] if insts else None
        if last and last[0] == "cc" and (last[1].startswith("s_branch") or last[1].startswith("s_cbranch")):
            tgt = last[2].split()[1]
            if tgt in index:
                s.append(index[tgt])
        if not (last and last[0] == "cc" and (last[1] == "s_branch" or last[1] == "s_endpgm")) and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    entry = [None] * len(blocks)
    entry[0] = ()
    work = [0]
    while work:
        i = work.pop()
        out = transfer(entry[i], blocks[i][1])
        for j in succ[i]:
            new = out if entry[j] is None else merge(entry[j], out)
            if new != entry[j]:
                entry[j] = new
                work.append(j)
    bad = []
    for i, (lab, insts) in enumerate(blocks):
        if entry[i] is not None:
            transfer(entry[i], insts, bad)
    return bad


def kernels(text):
    """(name, body) of every kernel function in the assembly."""
    names = re.findall(r"^(_Z\w+):\s", text, flags=re.M)
    out = []
    for n in names:
        start = text.index(f"\n{n}:")
        end = text.index(".Lfunc_end", start)
        out.append((n, text[start:end]))
    return out


def asm_lds_reads(body):
    """Number of inline-asm LDS reads in a kernel body."""
    return sum(1 for _, insts in parse(body) for k, op, _, _ in insts if k == "asm" and op.startswith("ds_read"))
