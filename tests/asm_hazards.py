"""Check of the compiled gfx950 assembly of the library's own kernels.

The GEMM cores issue their LDS transpose reads (ds_read_b64_tr_b16) as
inline assembly, so that the compiler does not order them behind the
direct-to-LDS loads in flight; their results are only valid after an
explicit lgkmcnt wait.  The compiler, which sees an asm output as defined at
once, must therefore not read, copy or reuse a destination register of such
a read on any path before that wait: a late-arriving result would overwrite
a register the compiler had given to something else (even an address).

``hazards(asm_text)`` walks each function's basic blocks forward (a dataflow
over the control flow, state = the LDS-counted operations in flight, in
order; lgkmcnt(n) retires all but the newest n) and returns the
(read, offending instruction) pairs.
"""

import re


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


def _parse(line):
    line = line.split(";")[0].strip()
    if not line:
        return None, []
    parts = line.split(None, 1)
    ops = [o.strip() for o in re.split(r",(?![^\[]*\])", parts[1])] if len(parts) > 1 else []
    return parts[0], ops


def _function_hazards(body):
    blocks, cur = [], []
    for l in body:
        if re.match(r"^\.LBB\S+:", l) and cur:
            blocks.append(cur)
            cur = []
        cur.append(l)
        if re.match(r"s_(cbranch|branch|setpc|endpgm)", l.strip()):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    labels = {}
    for bi, b in enumerate(blocks):
        for l in b:
            if re.match(r"^\.LBB\S+:", l):
                labels[l.split(":")[0]] = bi
    succ = []
    for bi, b in enumerate(blocks):
        op, ops = _parse(b[-1].strip())
        if op and op.startswith("s_branch"):
            s = [labels.get(ops[0])]
        elif op and op.startswith("s_cbranch"):
            s = [labels.get(ops[0]), bi + 1]
        elif op and (op.startswith("s_endpgm") or op.startswith("s_setpc")):
            s = []
        else:
            s = [bi + 1]
        succ.append([x for x in s if x is not None and x < len(blocks)])
    state_in = {0: ()}
    work = [0]
    found = set()
    while work:
        bi = work.pop()
        state = list(state_in[bi])
        in_asm = False
        for l in blocks[bi]:
            t = l.strip()
            if t.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if t.startswith(";;#ASMEND"):
                in_asm = False
                continue
            op, ops = _parse(t)
            if not op or op.startswith("."):
                continue
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", t)
                if m:
                    n = int(m.group(1))
                    state = [] if n == 0 else state[max(0, len(state) - n):]
                continue
            touched = frozenset()
            for o in ops:
                touched |= _regs(o)
            for dst, tag in state:
                if dst & touched:
                    found.add((tag, t))
            if op.startswith("ds_") or op.startswith("s_load") or op.startswith("s_buffer_load"):
                dst = _regs(ops[0]) if (in_asm and op.startswith("ds_read")) else frozenset()
                state.append((dst, t))
        for s in succ[bi]:
            new = tuple(state)
            old = state_in.get(s)
            if old is None:
                state_in[s] = new
                work.append(s)
            else:
                merged = tuple(dict.fromkeys(old + new))
                if len(merged) > len(old):
                    state_in[s] = merged
                    work.append(s)
    return found


def hazards(asm_text):
    """{(function, read, offending instruction)} over every function."""
    out = set()
    fn, body = None, []
    for l in asm_text.split("\n"):
        m = re.match(r"^(_Z\S+):", l)
        if m:
            fn, body = m.group(1), []
            continue
        if fn is None:
            continue
        body.append(l)
        if l.strip().startswith("s_endpgm"):
            out |= {(fn, a, b) for a, b in _function_hazards(body)}
            fn, body = None, []
    return out


def count_asm_reads(asm_text):
    n, in_asm = 0, False
    for l in asm_text.split("\n"):
        t = l.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
        elif t.startswith(";;#ASMEND"):
            in_asm = False
        elif in_asm and t.startswith("ds_read"):
            n += 1
    return n
