"""Static check of gfx950 assembly for loads issued from inline assembly.

A kernel that issues `global_load` through inline assembly (to keep a register ring
of prefetches in flight across loop iterations) hides those loads from the
compiler: to it the destination registers hold their value as soon as the asm
statement ends.  If it then reads, copies, spills or reuses such a register before
the explicit `s_waitcnt vmcnt(N)` that retires the load, the late write from memory
corrupts whatever the register holds by then (an address, a loop counter, a spilled
value).

This module walks the control-flow graph of every kernel in a `.s` file, models the
in-order vector-memory counter (every global/buffer/flat/scratch access increments
it; `s_waitcnt vmcnt(N)` retires the oldest until N remain), and reports each
instruction that touches a register an inline-assembly load is still writing.
Loads the compiler emitted itself are counted but not flagged: the compiler inserts
their waits.  Global-to-LDS loads (`global_load_lds_*`) write no register, so they
only count.  It also counts indirect register indexing (`movrel`, `s_set_gpr_idx`),
which inline-asm destinations cannot survive, and lists compiler-generated uses of
m0 in kernels whose inline assembly sets m0 for global-to-LDS loads (the compiler
treats m0 as reserved and may not honour a clobber of it).
"""
import re
from collections import defaultdict

_REG = re.compile(r'(?<![\w])([va])(?:\[(\d+):(\d+)\]|(\d+)(?![\w]))')
_VMEM = re.compile(r'(global|buffer|flat|scratch)_(load|store|atomic)')


def regs_of(text):
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            for i in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add((kind, i))
    return frozenset(out)


def split_kernels(text):
    """{symbol: [lines]} for every function body in an assembly file."""
    kernels, cur = {}, None
    for ln in text.split('\n'):
        m = re.match(r'^(_Z\S+):\s*(;.*)?$', ln)
        if m:
            cur = m.group(1)
            kernels[cur] = []
            continue
        if cur is not None and re.match(r'^\s*\.Lfunc_end', ln):
            cur = None
            continue
        if cur is not None:
            kernels[cur].append(ln)
    return kernels


def _blocks(lines):
    """Basic blocks [(label, [(instruction, from_asm)])] and successor lists."""
    items, in_asm = [], False
    for ln in lines:
        if ';;#ASMSTART' in ln:
            in_asm = True
        if ';;#ASMEND' in ln:
            in_asm = False
        s = ln.split(';')[0].rstrip()
        if not s.strip():
            continue
        m = re.match(r'^(\.L\w+):', s)
        if m:
            items.append(('label', m.group(1)))
        elif not s.strip().startswith('.'):
            items.append(('ins', (s.strip(), in_asm)))
    blocks, cur = [], ('<entry>', [])
    for kind, x in items:
        if kind == 'label':
            blocks.append(cur)
            cur = (x, [])
            continue
        cur[1].append(x)
        op = x[0].split()[0]
        if op.startswith('s_branch') or op.startswith('s_cbranch') or op == 's_endpgm':
            blocks.append(cur)
            cur = ('<after %d>' % len(blocks), [])
    blocks.append(cur)
    index = {lab: i for i, (lab, _) in enumerate(blocks)}
    succ = defaultdict(list)
    for i, (_, ins) in enumerate(blocks):
        last = ins[-1][0] if ins else ''
        op = last.split()[0] if last else ''
        if op == 's_endpgm':
            continue
        if op.startswith('s_branch'):
            succ[i].append(index[last.split()[1]])
            continue
        if op.startswith('s_cbranch'):
            succ[i].append(index[last.split()[1]])
        if i + 1 < len(blocks):
            succ[i].append(i + 1)
    return blocks, succ


def kernel_hazards(lines, max_states=256):
    """Instructions that touch an inline-asm load destination before its wait.

    The state carried along the control-flow graph is the list of outstanding
    vector-memory operations, oldest first, from the oldest inline-asm register load
    on: an entry is that load's destination registers, or None for any other
    operation (only its place in the order matters).  Operations older than every
    inline-asm load cannot change when such a load retires, so they are dropped.
    """
    blocks, succ = _blocks(lines)
    hazards = []
    seen = defaultdict(set)
    work = [(0, ())]
    while work:
        bi, state = work.pop()
        if state in seen[bi] or len(seen[bi]) >= max_states:
            continue
        seen[bi].add(state)
        pending = list(state)
        for ins, from_asm in blocks[bi][1]:
            op = ins.split()[0]
            operands = ins[len(op):]
            if op.startswith('s_waitcnt'):
                m = re.search(r'vmcnt\((\d+)\)', ins)
                if m:
                    keep = int(m.group(1))
                    while len(pending) > keep:
                        pending.pop(0)
                    while pending and pending[0] is None:
                        pending.pop(0)
                continue
            if pending:
                touched = regs_of(operands)
                for dest in pending:
                    if dest is not None and touched & dest:
                        hazards.append((ins, op))
            vm = _VMEM.match(op)
            if vm:
                loads = vm.group(2) == 'load' or (vm.group(2) == 'atomic' and 'glc' in ins)
                if '_lds_' in op:
                    loads = False   # writes LDS at m0; its first operand is the address
                if from_asm and loads:
                    pending.append(regs_of(operands.split(',')[0]))
                elif pending:
                    pending.append(None)
        nxt = tuple(pending)
        for s in succ[bi]:
            work.append((s, nxt))
    return hazards


def m0_writers(lines):
    """Instructions other than the inline-asm `s_mov_b32 m0, ...` that name m0."""
    out, in_asm = [], False
    for ln in lines:
        if ';;#ASMSTART' in ln:
            in_asm = True
        elif ';;#ASMEND' in ln:
            in_asm = False
        else:
            s = ln.split(';')[0]
            if re.search(r'\bm0\b', s) and not in_asm:
                out.append(s.strip())
    return out


def indirect_indexing(lines):
    return sum(1 for ln in lines if re.search(r'\b(v_movrel\w*|s_movrel\w*|s_set_gpr_idx\w*)', ln))


def has_asm_loads(lines):
    in_asm = False
    for ln in lines:
        if ';;#ASMSTART' in ln:
            in_asm = True
        elif ';;#ASMEND' in ln:
            in_asm = False
        elif in_asm and _VMEM.search(ln):
            return True
    return False
