"""Build-time check of the attention kernel's hand-issued bias loads.

The kernels that add a materialised [.., Q, K] bias issue its loads as
inline assembly (the compiler would otherwise wait for every in-flight LDS
copy before their first use) and retire them with an explicit vmcnt wait
whose operands are the loaded registers. The compiler treats an asm output
as ready when the statement ends, so nothing may read or write those
registers between the load and the wait that retires it. This module checks
that on the compiler's own output: a dataflow pass over the basic blocks of
each such kernel in the gfx950 assembly, tracking for every pending load how
many vector-memory operations were issued after it (a wait vmcnt(N) retires
the loads that are N or more operations old).
"""
from __future__ import annotations

import re

_BIAS_LOAD = re.compile(r"buffer_load_dwordx4 v\[(\d+):(\d+)\], v\d+, s\[\d+:\d+\], 0 offen$")
_LABEL = re.compile(r"^\.LBB\d+_\d+:")
_KERNEL = re.compile(r"^(_ZN3qfa\S*attn_fwd_kernel\S*ELb1EEEvNS_8AttnArgsEii):")   # last template flag: BIAS2D


def _regs(t: str) -> set[int]:
    r: set[int] = set()
    for a, c in re.findall(r"v\[(\d+):(\d+)\]", t):
        r |= set(range(int(a), int(c) + 1))
    for a in re.findall(r"(?<![\w\[:])v(\d+)\b", t):
        r.add(int(a))
    return r


def _check_function(ins: list[str]) -> list[tuple[str, str]]:
    blocks, cur = [], []
    for t in ins:
        if _LABEL.match(t):
            if cur:
                blocks.append(cur)
            cur = [t]
            continue
        cur.append(t)
        if t.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    labels = {b[0][:-1]: i for i, b in enumerate(blocks) if _LABEL.match(b[0])}
    succ = []
    for i, b in enumerate(blocks):
        m = re.match(r"s_(c?)branch\w* (\.LBB\d+_\d+)", b[-1])
        s = []
        if m:
            s.append(labels[m.group(2)])
            if m.group(1) == "c" and i + 1 < len(blocks):
                s.append(i + 1)
        elif not b[-1].startswith("s_endpgm") and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    state_in: list[frozenset | None] = [None] * len(blocks)
    state_in[0] = frozenset()
    work, bad = [0], set()
    while work:
        i = work.pop()
        state: dict[tuple, int] = {}
        for regs, age in state_in[i]:
            state[regs] = min(age, state.get(regs, 1 << 30))
        for t in blocks[i]:
            if _LABEL.match(t):
                continue
            m = _BIAS_LOAD.match(t)
            own = tuple(range(int(m.group(1)), int(m.group(2)) + 1)) if m else None
            used = _regs(t)
            for regs in state:
                if set(regs) & used and regs != own:
                    bad.add((blocks[i][0], t))
            if t.startswith(("buffer_", "global_")):
                state = {r: a + 1 for r, a in state.items()}
            if own:
                state[own] = 0
            w = re.search(r"vmcnt\((\d+)\)", t) if t.startswith("s_waitcnt") else None
            if w:
                n = int(w.group(1))
                state = {r: a for r, a in state.items() if a < n}
        out = frozenset(state.items())
        for s in succ[i]:
            new = out if state_in[s] is None else state_in[s] | out
            if new != state_in[s]:
                state_in[s] = new
                work.append(s)
    return sorted(bad)


def check(asm_path: str) -> dict[str, list[tuple[str, str]]]:
    """{kernel symbol: [(block, instruction) touching a pending bias load]} for every BIAS2D
    kernel in a gfx950 assembly file (empty lists when the property holds)."""
    lines = open(asm_path).read().split("\n")
    out = {}
    for k, line in enumerate(lines):
        m = _KERNEL.match(line)
        if not m:
            continue
        ins = []
        for t in lines[k + 1:]:
            if t.startswith(".Lfunc_end"):
                break
            t = t.split(";")[0].strip()
            if t and (not t.startswith(".") or _LABEL.match(t)):
                ins.append(t)
        out[m.group(1)] = _check_function(ins)
    return out
