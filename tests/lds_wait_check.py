"""Soundness check of the GEMM's hand-placed LDS waits, on the generated
gfx950 assembly.

The GEMM reads its MFMA fragments from LDS with inline-asm ds_read
instructions (the compiler cannot see them, so it does not wait on the LDS
copies in flight for them) and retires them with explicit
``s_waitcnt lgkmcnt(N)``.  That is only correct if no other instruction reads
or writes a destination register of such a read before a wait retires it.
This module checks exactly that, as a forward dataflow over the kernel's
basic blocks: the state is the ordered list of in-flight reads (oldest
first), ``lgkmcnt(N)`` keeps the newest N, and states meeting at a block
entry are merged position-wise from the newest end (a register stays
pending if it is pending on any path).
"""
from __future__ import annotations

import re

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_BRANCH_END = ("s_branch", "s_endpgm", "s_setpc_b64")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _parse(lines):
    """Basic blocks [label, [(is_asm, text)], successors] of one function body."""
    insts, in_asm = [], False
    for ln in lines:
        st = ln.strip()
        if st == ";;#ASMSTART":
            in_asm = True
            continue
        if st == ";;#ASMEND":
            in_asm = False
            continue
        s = st.split(";")[0].strip()
        if not s:
            continue
        if re.match(r"^\.?\w+:$", s):
            insts.append(("label", s[:-1]))
            continue
        if s.startswith("."):
            continue
        insts.append(("asm" if in_asm else "inst", s))
    blocks, cur = [], ["<entry>", []]
    for kind, s in insts:
        if kind == "label":
            blocks.append(cur)
            cur = [s, []]
            continue
        cur[1].append((kind == "asm", s))
        op = s.split()[0]
        if op.startswith("s_cbranch") or op in _BRANCH_END:
            blocks.append(cur)
            cur = ["<after %d>" % len(blocks), []]
    blocks.append(cur)
    names = [b[0] for b in blocks]
    out = []
    for i, (name, body) in enumerate(blocks):
        succ = []
        last = body[-1][1] if body else ""
        op = last.split()[0] if last else ""
        if op.startswith("s_cbranch") or op == "s_branch":
            tgt = last.split()[1]
            if tgt in names:
                succ.append(names.index(tgt))
        if op not in _BRANCH_END and i + 1 < len(blocks):
            succ.append(i + 1)
        out.append((name, body, succ))
    return out


def _merge(a, b):
    n = max(len(a), len(b))
    res = []
    for i in range(n, 0, -1):
        s = set()
        if len(a) >= i:
            s |= a[-i]
        if len(b) >= i:
            s |= b[-i]
        res.append(frozenset(s))
    return res


def _run(state, body, report):
    st = list(state)
    for is_asm, s in body:
        op = s.split()[0]
        m = re.search(r"lgkmcnt\((\d+)\)", s)
        if op == "s_waitcnt" and m:
            n = int(m.group(1))
            st = st[len(st) - n:] if len(st) > n else st
            continue
        pend = set().union(*st) if st else set()
        if is_asm and op.startswith("ds_read"):
            dst, addr = s.split(None, 1)[1].split(",", 1)
            if report is not None and (_regs(addr) & pend or _regs(dst) & pend):
                report.append("asm read touches an in-flight register: " + s)
            st.append(frozenset(_regs(dst)))
            continue
        if is_asm:
            continue
        if report is not None and st and (op.startswith("s_load") or op.startswith("s_buffer_load")):
            report.append("scalar load while LDS reads are in flight: " + s)
        args = s.split(None, 1)[1] if " " in s else ""
        hit = _regs(args) & pend
        if hit and report is not None:
            report.append("touches in-flight %s: %s" % (sorted(hit)[:4], s))
    return st


def check_function(asm_text: str, name: str):
    """-> (violations, number of inline-asm LDS reads) for function `name`."""
    lines = asm_text.split("\n")
    i0 = next(i for i, l in enumerate(lines) if l.startswith(name + ":"))
    i1 = next(i for i in range(i0, len(lines)) if lines[i].startswith(".Lfunc_end"))
    blocks = _parse(lines[i0 + 1:i1])
    ins, outs, work = {0: []}, {}, [0]
    while work:
        b = work.pop()
        o = _run(ins[b], blocks[b][1], None)
        if outs.get(b) == o:
            continue
        outs[b] = o
        for sj in blocks[b][2]:
            new = _merge(ins[sj], o) if sj in ins else o
            if ins.get(sj) != new:
                ins[sj] = new
                work.append(sj)
    report = []
    for b in ins:
        _run(ins[b], blocks[b][1], report)
    nreads = sum(1 for _, body, _ in blocks for a, s in body if a and s.startswith("ds_read"))
    return report, nreads


def gemm_functions(asm_text: str):
    """The kernels that run the GEMM mainloop: k_gemm and the fused k_mega."""
    return [m.group(1) for m in re.finditer(r"^(_ZN2mm6k_(?:gemm|mega)\w+):", asm_text, flags=re.M)]
