"""Path-sensitive check of MFMA result hazards in gfx950 assembly (test
infrastructure: it reads the device assembly that hipcc writes for this
repository's own kernel sources).

On CDNA the hardware does not stall a VALU, LDS or global-memory instruction
that reads a VGPR an in-flight MFMA is still writing: the compiler has to leave
enough independent instructions ("wait states", s_nop n counting n + 1)
between them.  The compiler emits those waits along the straight-line
(fall-through) order; this module walks every control-flow path backwards
from each reader and reports the fewest wait states on any path, so a branch
that jumps over the padding shows up.
"""
from __future__ import annotations

import re
from collections import defaultdict

_VR = re.compile(r'^v\[(\d+):(\d+)\]$|^v(\d+)$')


def vregs(tok: str) -> frozenset:
    m = _VR.match(tok.strip())
    if not m:
        return frozenset()
    if m.group(3) is not None:
        return frozenset((int(m.group(3)),))
    return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))


def functions(asm: str):
    """(name, body lines) of every kernel in an assembly file."""
    lines = asm.split('\n')
    for i, l in enumerate(lines):
        m = re.match(r'^(_Z\S+):', l)
        if m:
            end = next(j for j in range(i, len(lines)) if lines[j].startswith('.Lfunc_end'))
            yield m.group(1), lines[i + 1:end]


class Inst:
    __slots__ = ('op', 'args', 'ws', 'mfma', 'dst', 'reads')

    def __init__(self, text: str):
        op, _, rest = text.partition(' ')
        self.op = op
        self.args = [a.strip() for a in rest.split(',')] if rest.strip() else []
        self.ws = int(self.args[0], 0) + 1 if op == 's_nop' else 1
        self.mfma = op.startswith('v_mfma')
        a = self.args
        if self.mfma:
            self.dst = vregs(a[0])
            self.reads = vregs(a[1]) | vregs(a[2]) | (vregs(a[3]) if len(a) > 3 else frozenset())
        elif op.startswith(('global_store', 'buffer_store', 'ds_write', 'flat_store', 'scratch_store')):
            self.dst = frozenset()
            self.reads = frozenset().union(*[vregs(x) for x in a]) if a else frozenset()
        elif op.startswith(('v_', 'ds_', 'global_', 'buffer_', 'flat_', 'scratch_')):
            self.dst = vregs(a[0]) if a else frozenset()
            self.reads = frozenset().union(*[vregs(x) for x in a[1:]]) if len(a) > 1 else frozenset()
        else:
            self.dst = frozenset()
            self.reads = frozenset()


def blocks_of(body):
    """Basic blocks [(label, [Inst])] and predecessor lists."""
    blocks = [('entry', [])]
    for l in body:
        t = l.split(';')[0].strip()
        c = l.strip()
        if c.startswith('; %bb.'):
            blocks.append((c[2:].split()[0], []))
            continue
        if not t:
            continue
        if t.startswith('.LBB') and t.endswith(':'):
            blocks.append((t[:-1], []))
            continue
        if t.startswith('.'):
            continue
        blocks[-1][1].append(Inst(t))
    idx = {b[0]: i for i, b in enumerate(blocks)}
    preds = defaultdict(list)
    for i, (_, ins) in enumerate(blocks):
        last = ins[-1] if ins else None
        op = last.op if last else ''
        if op.startswith('s_cbranch') or op == 's_branch':
            if last.args and last.args[0] in idx:
                preds[idx[last.args[0]]].append(i)
        if op not in ('s_branch', 's_endpgm', 's_setpc_b64') and i + 1 < len(blocks):
            preds[i + 1].append(i)
    return blocks, preds


def raw_distances(body, limit=32):
    """For every non-MFMA instruction reading a VGPR that an MFMA wrote: the
    fewest wait states between them over every path, and that over the
    fall-through order alone.  Yields (mfma opcode, min any path, min
    fall-through, reader text)."""
    blocks, preds = blocks_of(body)
    for bi, (_, ins) in enumerate(blocks):
        for ii, r in enumerate(ins):
            if r.mfma or not r.reads:
                continue
            best_any = {}
            best_ft = {}
            # (block, index, wait states, fall-through only so far)
            stack = [(bi, ii - 1, 0, True)]
            seen = set()
            while stack:
                b, j, w, ft = stack.pop()
                if w > limit or (b, j, w, ft) in seen:
                    continue
                seen.add((b, j, w, ft))
                if j < 0:
                    for p in preds[b]:
                        stack.append((p, len(blocks[p][1]) - 1, w, ft and p == b - 1))
                    continue
                u = blocks[b][1][j]
                if u.mfma and (u.dst & r.reads):
                    if w < best_any.get(u.op, 99):
                        best_any[u.op] = w
                    if ft and w < best_ft.get(u.op, 99):
                        best_ft[u.op] = w
                    continue
                stack.append((b, j - 1, w + u.ws, ft))
            for op, w in best_any.items():
                yield op, w, best_ft.get(op, 99), r.op + ' ' + ','.join(r.args)
