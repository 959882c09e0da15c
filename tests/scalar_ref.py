"""Scalar per-thread reference for the PTX subset (tests only).

Each thread runs alone, one instruction at a time, with plain control flow (a
taken branch jumps, ret stops the thread).  For race-free programs whose
barriers sit at converged points this gives the same final memory as any
correct SIMT execution, and the number of instructions each thread executes
is its own path length.  It models no warps, no cycles and no analyser, so it
pins the oracle's values and thread-instruction totals independently of the
divergence stack.
"""
import re

import numpy as np

from . import ieee32

_REG = re.compile(r"\.reg\s+\.(\w+)\s+(.+)")


def _ints(s):
    s = s.strip()
    neg = s.startswith("-")
    if neg:
        s = s[1:]
    v = int(s, 16) if s.lower().startswith("0x") else int(s)
    return -v if neg else v


class Program:
    def __init__(self, ptx):
        text = re.sub(r"//[^\n]*", "", ptx)
        body = text[text.index("{") + 1: text.rindex("}")]
        head = text[: text.index("{")]
        self.params = []
        off = 0
        for m in re.finditer(r"\.param\s+\.(\w+)\s+(\w+)", head):
            size = 8 if m.group(1)[1:] == "64" else 4
            off = (off + size - 1) // size * size
            self.params.append((m.group(2), off, size))
            off += size
        self.width = {}
        self.shared = {}
        shoff = 0
        self.code = []
        self.labels = {}
        for raw in body.split("\n"):
            line = raw.strip()
            if not line or line.startswith(".loc"):
                continue
            while True:
                m = re.match(r"^([\w$]+):\s*(.*)$", line)
                if not m:
                    break
                self.labels[m.group(1)] = len(self.code)
                line = m.group(2)
            if not line:
                continue
            line = line.rstrip(";").strip()
            if line.startswith(".reg"):
                m = _REG.match(line)
                t = m.group(1)
                w = 1 if t == "pred" else (64 if t.endswith("64") else 32)
                for nm in m.group(2).split(","):
                    nm = nm.strip()
                    r = re.match(r"(%\w+)<(\d+)>", nm)
                    if r:
                        for k in range(int(r.group(2))):
                            self.width[r.group(1) + str(k)] = w
                    else:
                        self.width[nm] = w
                continue
            if line.startswith(".shared"):
                m = re.search(r"\.(\w+)\s+(\w+)\[(\d+)\]", line)
                al = re.search(r"\.align\s+(\d+)", line)
                esz = {"b8": 1, "b16": 2, "b32": 4, "b64": 8}[m.group(1)]
                a = int(al.group(1)) if al else esz
                shoff = (shoff + a - 1) // a * a
                self.shared[m.group(2)] = shoff
                shoff += esz * int(m.group(3))
                continue
            guard = None
            m = re.match(r"^@(!?)(%\w+)\s+(.*)$", line)
            if m:
                guard = (m.group(1) == "!", m.group(2))
                line = m.group(3)
            parts = line.split(None, 1)
            opw = parts[0]
            ops = [o.strip() for o in re.split(r",(?![^\[]*\])", parts[1])] if len(parts) > 1 else []
            self.code.append((guard, opw.split("."), ops))
        self.shared_bytes = shoff


def _f32_bits(x):
    return int(np.float32(x).view(np.uint32))


def run_thread(prog, params, gmem, shared, tid3, ntid3, ctaid3, nctaid3, laneid, max_steps=1 << 22):
    regs = {}
    n = len(prog.code)
    pc = 0
    steps = 0
    special = {"%tid.x": tid3[0], "%tid.y": tid3[1], "%tid.z": tid3[2], "%ntid.x": ntid3[0],
               "%ntid.y": ntid3[1], "%ntid.z": ntid3[2], "%ctaid.x": ctaid3[0], "%ctaid.y": ctaid3[1],
               "%ctaid.z": ctaid3[2], "%nctaid.x": nctaid3[0], "%nctaid.y": nctaid3[1],
               "%nctaid.z": nctaid3[2], "%laneid": laneid}

    def val(o, width):
        if o in prog.width:
            return regs.get(o, 0)
        if o in special:
            return special[o]
        if o in prog.shared:
            return prog.shared[o]
        if o[:2] in ("0f", "0F"):
            return int(o[2:], 16)
        return _ints(o) & ((1 << width) - 1)

    def addr(o):
        o = o.strip("[]").strip()
        m = re.match(r"^(%?[\w$]+)\s*([+-])?\s*(\w+)?$", o)
        base, sign, off = m.group(1), m.group(2), m.group(3)
        d = _ints(off) if off else 0
        if sign == "-":
            d = -d
        return base, d

    def mem_valid(a, size, limit):
        return a % size == 0 and 0 <= a and a + size <= limit

    while pc < n and steps < max_steps:
        guard, parts, ops = prog.code[pc]
        steps += 1
        nxt = pc + 1
        ok = True
        if guard is not None:
            ok = bool(regs.get(guard[1], 0)) != guard[0]
        base = parts[0]
        typ = parts[-1]
        w = 64 if typ.endswith("64") else 32
        mask = (1 << w) - 1
        if ok:
            if base in ("add", "sub") and typ == "f32":
                a, b = val(ops[1], 32), val(ops[2], 32)
                regs[ops[0]] = ieee32.add(a, b) if base == "add" else ieee32.sub(a, b)
            elif base == "mul" and typ == "f32":
                regs[ops[0]] = ieee32.mul(val(ops[1], 32), val(ops[2], 32))
            elif base == "fma":
                regs[ops[0]] = ieee32.fma(val(ops[1], 32), val(ops[2], 32), val(ops[3], 32))
            elif base == "add":
                regs[ops[0]] = (val(ops[1], w) + val(ops[2], w)) & mask
            elif base == "sub":
                regs[ops[0]] = (val(ops[1], w) - val(ops[2], w)) & mask
            elif base == "mul" and parts[1] == "lo":
                regs[ops[0]] = (val(ops[1], w) * val(ops[2], w)) & mask
            elif base == "mul" and parts[1] == "wide":
                a, b = val(ops[1], 32), val(ops[2], 32)
                if typ == "s32":
                    a = a - (1 << 32) if a >> 31 else a
                    b = b - (1 << 32) if b >> 31 else b
                regs[ops[0]] = (a * b) & ((1 << 64) - 1)
            elif base == "mad":
                regs[ops[0]] = (val(ops[1], w) * val(ops[2], w) + val(ops[3], w)) & mask
            elif base == "setp":
                cmp = parts[1]
                a, b = val(ops[1], w), val(ops[2], w)
                if typ == "f32":
                    ka, _, va = ieee32.classify(a)
                    kb, _, vb = ieee32.classify(b)
                    if ka == "nan" or kb == "nan":
                        r = False
                    else:
                        fa = va if ka == "num" else (float("-inf") if a >> 31 else float("inf"))
                        fb = vb if kb == "num" else (float("-inf") if b >> 31 else float("inf"))
                        r = {"eq": fa == fb, "ne": fa != fb, "lt": fa < fb, "le": fa <= fb,
                             "gt": fa > fb, "ge": fa >= fb}[cmp]
                else:
                    if typ[0] == "s":
                        a = a - (1 << w) if a >> (w - 1) else a
                        b = b - (1 << w) if b >> (w - 1) else b
                    cmp = {"lo": "lt", "ls": "le", "hi": "gt", "hs": "ge"}.get(cmp, cmp)
                    r = {"eq": a == b, "ne": a != b, "lt": a < b, "le": a <= b, "gt": a > b,
                         "ge": a >= b}[cmp]
                regs[ops[0]] = 1 if r else 0
            elif base == "selp":
                regs[ops[0]] = val(ops[1], w) if regs.get(ops[3], 0) else val(ops[2], w)
            elif base == "mov":
                regs[ops[0]] = val(ops[1], w)
            elif base == "ld" and parts[1] == "param":
                name, d = addr(ops[1])
                for pn, po, ps in prog.params:
                    if pn == name:
                        regs[ops[0]] = int.from_bytes(params[po + d: po + d + w // 8], "little")
            elif base in ("ld", "st"):
                space = parts[1]
                memo = ops[1] if base == "ld" else ops[0]
                rname, d = addr(memo)
                rv = regs.get(rname, 0)
                a = (rv + d) & ((1 << 64) - 1)
                buf = gmem if space == "global" else shared
                size = w // 8
                if mem_valid(a, size, len(buf)):
                    if base == "ld":
                        regs[ops[0]] = int.from_bytes(bytes(buf[a: a + size]), "little")
                    else:
                        v = regs.get(ops[1], 0) & mask
                        buf[a: a + size] = np.frombuffer(v.to_bytes(size, "little"), dtype=np.uint8)
                elif base == "ld":
                    regs[ops[0]] = 0
            elif base == "bra":
                nxt = prog.labels[ops[0]]
            elif base in ("ret", "exit"):
                return steps
            elif base == "bar":
                pass
            else:
                raise ValueError("scalar reference: unsupported %s" % ".".join(parts))
        pc = nxt
    return steps


def run_grid(ptx, grid, block, params, gmem, blocks=None):
    """Run every thread of the listed blocks (default: all) alone, in order.
    Returns the per-thread step counts, indexed [block position][thread]."""
    prog = Program(ptx)
    gx, gy, gz = grid
    bx, by, bz = block
    tpb = bx * by * bz
    out = []
    ids = range(gx * gy * gz) if blocks is None else blocks
    for bl in ids:
        ctaid = (bl % gx, (bl // gx) % gy, bl // (gx * gy))
        shared = np.zeros(max(prog.shared_bytes, 1), dtype=np.uint8)
        counts = []
        for t in range(tpb):
            tid = (t % bx, (t // bx) % by, t // (bx * by))
            counts.append(run_thread(prog, params, gmem, shared, tid, block, ctaid, grid, t % 32))
        out.append(counts)
    return out
