"""Check of compiled gfx9 device assembly: no instruction may read or write a
vector register that an inline-assembly vector-memory load is still writing.

The kernels issue some global loads as inline assembly and wait for them with
explicit ``s_waitcnt vmcnt(N)`` statements. The compiler does not see those
loads: if it copies or reuses a destination register before the wait (for
instance to merge the value of a conditional block with another definition),
the data lands later on top of an unrelated value. An address corrupted that
way faults the GPU.

Model. The assembly of each function is cut into basic blocks (labels,
branches). A forward dataflow over the control-flow graph tracks the vector
memory operations that may be outstanding at each point, each with its age
(the number of vector memory operations issued after it). Loads return in
issue order, so ``s_waitcnt vmcnt(N)`` retires every operation with age >= N.
An instruction that names a register of an outstanding inline-assembly load
(between ``;;#ASMSTART`` and ``;;#ASMEND``, LDS-destination loads excluded)
is reported. The states of a block are kept apart by the flag registers the
compiler uses to join the two arms of a branch (an SGPR pair set to 0 or -1,
turned into VCC and branched on), so that a path through neither arm is not
followed; otherwise the analysis is path-insensitive, and a branch on a
condition correlated with an earlier one (a loop's last iteration, say) can
produce a report on a path that never runs. It is applied to the kernels
whose code it clears.
"""
from __future__ import annotations

import re

_VMEM = re.compile(r"^(global_|buffer_|scratch_|flat_)(load|store|atomic)")
_VREG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")
_FUNC = re.compile(r"^(_Z\S+):")
_LABEL = re.compile(r"^(\.LBB\S+):$")


def _vregs(text):
    out = set()
    for m in _VREG.finditer(text):
        if m.group(1):
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return frozenset(out)


def parse(text):
    """{function: [(label, [(line, instruction, in_inline_asm)])]}"""
    funcs, cur, blk, inasm = {}, None, None, False
    for ln, raw in enumerate(text.splitlines(), 1):
        s = raw.strip()
        m = _FUNC.match(raw)
        if m:
            cur = m.group(1)
            blk = ["<entry>", []]
            funcs[cur] = [blk]
            continue
        if cur is None:
            continue
        if s.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if s.startswith(";;#ASMEND"):
            inasm = False
            continue
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        code = s.split(";")[0].strip()
        if not code:
            continue
        m = _LABEL.match(code)
        if m:
            blk = [m.group(1), []]
            funcs[cur].append(blk)
            continue
        if code.startswith("."):
            continue
        blk[1].append((ln, code, inasm))
        op = code.split()[0]
        if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm", "s_setpc_b64"):
            # a terminator ends the block; what follows is a block of its own
            # (reached by falling through a conditional branch)
            blk = [f"<after {ln}>", []]
            funcs[cur].append(blk)
    return funcs


def _successors(blocks):
    index = {b[0]: i for i, b in enumerate(blocks)}
    succ = []
    for i, (_, ins) in enumerate(blocks):
        nxt = [i + 1] if i + 1 < len(blocks) else []
        last = ins[-1][1] if ins else ""
        op = last.split()[0] if last else ""
        if op == "s_branch":
            succ.append([index[last.split()[1]]])
        elif op.startswith("s_cbranch"):
            succ.append([index[last.split()[1]]] + nxt)
        elif op in ("s_endpgm", "s_setpc_b64"):
            succ.append([])
        else:
            succ.append(nxt)
    return succ


_SREG = re.compile(r"^s\[(\d+):(\d+)\]$|^s(\d+)$")


def _sregs(tok):
    m = _SREG.match(tok)
    if not m:
        return frozenset()
    if m.group(3) is not None:
        return frozenset([int(m.group(3))])
    return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))


def _flags_after(code, flags, vcc):
    """Known flag facts after one instruction. A fact is an SGPR pair holding 0
    or -1 (``s_mov_b64``), or the outcome of an earlier branch on
    ``exec & sX`` / ``exec & ~sX``; VCC is "nz", "z", a pending test
    ("and"/"andn2", sX) or unknown. Exec is taken as non-empty: with no lane
    active no vector register changes."""
    toks = code.replace(",", " ").split()
    op = toks[0]
    facts = dict(flags)
    if op in ("s_andn2_b64", "s_and_b64") and len(toks) > 3 and toks[1] == "vcc" and toks[2] == "exec":
        r = tuple(sorted(_sregs(toks[3])))
        kind = "andn2" if op == "s_andn2_b64" else "and"
        v = facts.get(("const", r))
        if v is not None:
            on = (v == 0) if kind == "andn2" else (v == -1)
            return frozenset(facts.items()), ("nz" if on else "z")
        return frozenset(facts.items()), facts.get((kind, r), (kind, r))
    written = set()
    for t in toks[1:3] if op.startswith("v_") else toks[1:2]:
        written |= _sregs(t)
    if written:
        facts = {k: v for k, v in facts.items() if not (set(k[1]) & written)}
    if "exec" in toks[1:2] or "saveexec" in op or op.startswith("v_cmpx"):
        facts = {k: v for k, v in facts.items() if k[0] == "const"}
    if "vcc" in toks[1:3] or op.startswith("v_cmp") or "_co_" in op or "vcc" in op:
        vcc = None
    if op == "s_mov_b64" and _sregs(toks[1]) and toks[2] in ("0", "-1"):
        facts[("const", tuple(sorted(_sregs(toks[1]))))] = int(toks[2])
    return frozenset(facts.items()), vcc


def _exec_after(code, ex):
    """Exec after one instruction: "ne" (some lane active), "e" (none), None."""
    toks = code.replace(",", " ").split()
    op = toks[0]
    if op == "s_or_b64" and toks[1:3] == ["exec", "exec"]:
        return "ne" if ex == "ne" else None  # a join restores at least the lanes it had
    if "exec" in toks[1:2] or "saveexec" in op or op.startswith("v_cmpx"):
        return None
    return ex


_MAX_KEYS = 64  # distinct flag states kept per block before they are merged


def check_function(blocks):
    """[(line, instruction, line of the load, registers)] of one function."""
    succ = _successors(blocks)
    # per block: {(known flags, vcc, exec): {load line: (age, destination registers, inline asm)}}
    state_in = [dict() for _ in blocks]
    start = (frozenset(), None, "ne")
    state_in[0][start] = {}
    found = {}
    work = [(0, start)]
    while work:
        i, key = work.pop()
        consts, vcc, ex = key
        st = dict(state_in[i][key])
        term = None
        for ln, code, inasm in blocks[i][1]:
            op = code.split()[0]
            ops = code[len(op):]
            if op == "s_waitcnt":
                m = re.search(r"vmcnt\((\d+)\)", code)
                if m:
                    n = int(m.group(1))
                    st = {k: v for k, v in st.items() if v[0] < n}
                elif re.match(r"s_waitcnt\s+0\s*$", code):
                    st = {}
                continue
            if op.startswith("s_cbranch") or op == "s_branch":
                term = op
                continue
            used = _vregs(ops) if ex != "e" else frozenset()  # no lane: no register changes
            for k, (age, dst, asm) in st.items():
                if asm and dst & used:
                    found.setdefault(ln, (code, k, sorted(dst & used)))
            if _VMEM.match(op):
                st = {k: (min(a + 1, 64), d, x) for k, (a, d, x) in st.items()}
                load = "load" in op and "lds" not in op and ex != "e"
                st[ln] = (0, _vregs(ops.split(",")[0]) if load else frozenset(), inasm and load)
            consts, vcc = _flags_after(code, consts, vcc)
            ex = _exec_after(code, ex)
        edges = [(j, consts, vcc, ex) for j in succ[i]]
        if term in ("s_cbranch_vccnz", "s_cbranch_vccz") and vcc is not None and len(succ[i]) == 2:
            t, f = succ[i]
            if vcc in ("nz", "z"):
                taken = (vcc == "nz") == (term == "s_cbranch_vccnz")
                edges = [(t if taken else f, consts, vcc, ex)]
            else:  # a test of exec & sX: each edge learns its outcome
                on_t = "nz" if term == "s_cbranch_vccnz" else "z"
                on_f = "z" if on_t == "nz" else "nz"
                edges = [(t, consts | {(vcc, on_t)}, on_t, ex), (f, consts | {(vcc, on_f)}, on_f, ex)]
        elif term in ("s_cbranch_execz", "s_cbranch_execnz") and len(succ[i]) == 2:
            t, f = succ[i]
            on_t = "e" if term == "s_cbranch_execz" else "ne"
            on_f = "ne" if on_t == "e" else "e"
            edges = [(j, consts, vcc, e) for j, e in ((t, on_t), (f, on_f)) if not (ex == "ne" and e == "e")]
        for j, consts_j, vcc_j, ex_j in edges:
            out_key = (frozenset(consts_j), vcc_j, ex_j)
            if out_key not in state_in[j] and len(state_in[j]) >= _MAX_KEYS:
                out_key = (frozenset(), None, None)  # widen: nothing known about the flags
            cur = state_in[j].get(out_key)
            if cur is None:
                state_in[j][out_key] = dict(st)
                work.append((j, out_key))
                continue
            merged, changed = dict(cur), False
            for k, v in st.items():
                if k not in merged or v[0] < merged[k][0]:
                    merged[k] = v
                    changed = True
            if changed:
                state_in[j][out_key] = merged
                work.append((j, out_key))
    return [(ln, code, k, regs) for ln, (code, k, regs) in sorted(found.items())]


def check(text):
    """{function: findings} for every function with at least one finding."""
    out = {}
    for name, blocks in parse(text).items():
        f = check_function(blocks)
        if f:
            out[name] = f
    return out
