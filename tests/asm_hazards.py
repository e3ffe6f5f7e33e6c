"""Checks on the device assembly of the MFMA kernels (host-side, no GPU).

The kernels issue their LDS fragment reads and bf16 MFMAs as inline asm, so
the compiler neither tracks when a read's result lands nor applies its
hazard rules to the MFMAs' operands. Two rules the code must keep, checked
on the compiler's output over each kernel's control-flow graph:

* in-flight reads: no instruction may read or write a VGPR while an LDS
  read into it may still be outstanding (LDS reads complete in order; an
  ``s_waitcnt lgkmcnt(N)`` leaves at most the N newest outstanding);
* VALU to MFMA: an MFMA may not read a VGPR that a VALU instruction wrote
  fewer than two instructions earlier (the wait states the hardware does
  not enforce);
* store data: the instruction right after a global or buffer store of more
  than 8 bytes may not write the store's data registers (VGPRs or AGPRs:
  one wait state, which the compiler inserts for its own stores but not
  after asm ones).

``exec``-conditional branches are taken as always taken: every lane of
these kernels' waves is active.
"""
from __future__ import annotations

import re


def _regs(tok: str) -> frozenset:
    m = re.fullmatch(r'v\[(\d+):(\d+)\]', tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r'v(\d+)', tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


# AGPRs as register numbers 1000 and up (disjoint from the VGPRs)
def _va_regs(tok: str) -> frozenset:
    m = re.fullmatch(r'a\[(\d+):(\d+)\]', tok)
    if m:
        return frozenset(1000 + r for r in range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r'a(\d+)', tok)
    return frozenset({1000 + int(m.group(1))}) if m else _regs(tok)


def _split(line: str):
    parts = line.split(None, 1)
    ops = []
    if len(parts) > 1:
        body = parts[1].split(' offset:')[0]
        ops = [o.strip().split()[0] for o in re.split(r',\s*', body) if o.strip()]
    return parts[0], ops


def kernels(asm: str) -> dict:
    """name -> body text of every function in a device assembly file."""
    out = {}
    for m in re.finditer(r'^(\S+):\s*(?:;.*)?$', asm, flags=re.M):
        name = m.group(1)
        if name.startswith('.') or not name.startswith('_Z'):
            continue
        end = asm.find('.Lfunc_end', m.end())
        if end > 0:
            out[name] = asm[m.end():end]
    return out


def _cfg(body: str):
    blocks, order = {'entry': []}, ['entry']
    cur = 'entry'
    for raw in body.split('\n'):
        line = raw.split(';')[0].strip()
        if not line:
            continue
        m = re.match(r'^(\.LBB\d+_\d+):', line)
        if m:
            cur = m.group(1)
            blocks[cur] = []
            order.append(cur)
            continue
        if line.startswith('.'):
            continue
        blocks[cur].append(line)
    succ = {}
    for i, b in enumerate(order):
        nxt = order[i + 1] if i + 1 < len(order) else None
        last = blocks[b][-1] if blocks[b] else ''
        tgt = re.findall(r'(\.LBB\d+_\d+)', last)
        if last.startswith('s_branch'):
            s = tgt
        elif last.startswith('s_cbranch_execnz'):
            s = tgt
        elif last.startswith('s_cbranch_execz'):
            s = [nxt] if nxt else []
        elif last.startswith('s_cbranch'):
            s = tgt + ([nxt] if nxt else [])
        elif last.startswith('s_endpgm'):
            s = []
        else:
            s = [nxt] if nxt else []
        succ[b] = [t for t in s if t in blocks]
    return blocks, order, succ


def _merge(a, b):
    n = max(len(a), len(b))
    a = [frozenset()] * (n - len(a)) + list(a)
    b = [frozenset()] * (n - len(b)) + list(b)
    return tuple(x | y for x, y in zip(a, b))


def _solve(body: str, transfer) -> set:
    blocks, order, succ = _cfg(body)
    state = {b: None for b in order}
    state['entry'] = ()
    work, bad = ['entry'], set()
    while work:
        b = work.pop()
        st = tuple(state[b])
        for line in blocks[b]:
            st = transfer(st, line, lambda l, b=b: bad.add((b, l)))
        for t in succ[b]:
            new = st if state[t] is None else _merge(state[t], st)
            if state[t] is None or new != state[t]:
                state[t] = new
                work.append(t)
    return bad


def _inflight(st, line, report):
    op, ops = _split(line)
    if op.startswith('s_waitcnt'):
        m = re.search(r'lgkmcnt\((\d+)\)', line)
        if m:
            n = int(m.group(1))
            st = st[len(st) - n:] if n else ()
        return st
    pending = frozenset().union(*st) if st else frozenset()
    touched = frozenset().union(*[_regs(o) for o in ops]) if ops else frozenset()
    if touched & pending:
        report(line)
    if op.startswith('ds_read'):
        return tuple(st) + (_regs(ops[0]),)
    return st


def _valu_mfma(st, line, report):
    op, ops = _split(line)
    if op.startswith('v_mfma'):
        reads = frozenset().union(*[_regs(o) for o in ops[1:]]) if len(ops) > 1 else frozenset()
        if reads & (frozenset().union(*st) if st else frozenset()):
            report(line)
        new = frozenset()
    elif op.startswith('v_') and ops:
        new = _regs(ops[0])
    else:
        new = frozenset()
    return (tuple(st) + (new,))[-2:]


def _store_data(st, line, report):
    op, ops = _split(line)
    guarded = st[0] if st else frozenset()
    if op.startswith('s_nop'):
        return (frozenset(),)
    if op.startswith('v_') and ops and (_va_regs(ops[0]) & guarded):
        report(line)
    wide = op.endswith(('_dwordx3', '_dwordx4', '_b96', '_b128'))
    if wide and op.startswith('global_store') and len(ops) > 1:
        return (_va_regs(ops[1]),)
    if wide and op.startswith('buffer_store') and ops:
        return (_va_regs(ops[0]),)
    return (frozenset(),)


def check(asm: str, prefix: str = '') -> dict:
    """Violations of the rules per kernel whose name starts with `prefix`:
    {name: {"inflight": [...], "valu_mfma": [...], "store_data": [...]}}
    (empty lists: clean)."""
    out = {}
    for name, body in kernels(asm).items():
        if not name.startswith(prefix):
            continue
        out[name] = {"inflight": sorted(l for _, l in _solve(body, _inflight)),
                     "valu_mfma": sorted(l for _, l in _solve(body, _valu_mfma)),
                     "store_data": sorted(l for _, l in _solve(body, _store_data))}
    return out
