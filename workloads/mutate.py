"""Seeded mutations of valid programs (inputs only, no simulator arithmetic).

Each mutation keeps the text inside the subset's grammar but changes what the
program does: a register operand swapped for another declared register of the
same family, a guard negated, added or dropped, a branch sent to another label
(which can make loops), a `bar.sync 0` inserted anywhere (also inside divergent
code), a comparison changed, an immediate changed, a line duplicated or deleted.
A mutant can read registers no instruction wrote, loop until its issue budget,
diverge at barriers or fault; whether it is race-free is for the caller to check.
"""
import re

import numpy as np

from . import configs as W
from . import small as S
from .configs import Workload

CMPS = ["eq", "ne", "lt", "le", "gt", "ge"]
IMMS = [0, 1, 2, 3, 4, 7, 8, 31, 32, 33, 64, 255, 4096]


def base_programs():
    """The valid programs mutations start from."""
    return ([W.VECTOR_ADD_PTX, W.STRIDED_PTX, S.block_reduce_ptx(64), S.block_reduce_ptx(128), S.tile_transpose_ptx(1),
             S.stencil3_ptx(), S.lcg64_ptx(4), S.setp_forms_ptx(), S.f32_setp_ptx(), S.shared_edges_ptx(),
             S.staircase_ptx(7), S.fma_chain_ptx(9, 3)]
            + [S.random_cfg_ptx(s, n_instr=30, loops=bool(s % 2)) for s in range(12)])


def _decls(text):
    return {nm: (ty, int(n)) for ty, nm, n in re.findall(r"\.reg\s+\.(\w+)\s+(%\w+?)<(\d+)>", text)}


def mutate(rnd, text):
    """One to three mutations of `text`, drawn from the random.Random `rnd`."""
    lines = text.split("\n")
    regs = _decls(text)
    body = [i for i, ln in enumerate(lines)
            if re.match(r"\s+(@!?%p\d+\s+)?([a-z]+\.[\w.]*|bra|ret|bar)\b", ln) and not ln.strip().startswith(".")]
    labels = re.findall(r"^(\$?\w+):", text, re.M)
    if not body:
        return text
    for _ in range(rnd.randint(1, 3)):
        i = rnd.choice(body)
        ln = lines[i]
        kind = rnd.randrange(8)
        if kind == 0:  # another register of the same family
            names = re.findall(r"%[a-z]+\d+", ln)
            if names:
                r = rnd.choice(names)
                fam = re.match(r"(%[a-z]+)", r).group(1)
                if fam in regs:
                    ln = ln.replace(r, "%s%d" % (fam, rnd.randrange(regs[fam][1])), 1)
        elif kind == 1:  # guard negated, dropped or added
            m = re.match(r"(\s+)@(!?)(%p\d+)\s+(.*)", ln)
            if m:
                ln = m.group(1) + (m.group(4) if rnd.random() < 0.3 else
                                   "@%s%s %s" % ("" if m.group(2) else "!", m.group(3), m.group(4)))
            elif "%p" in regs and not ln.strip().startswith("ret"):
                ln = re.sub(r"^(\s+)", r"\1@%%p%d " % rnd.randrange(regs["%p"][1]), ln, count=1)
        elif kind == 2 and labels:  # another branch target
            ln = re.sub(r"bra(\.uni)?\s+\$?\w+;", "bra %s;" % rnd.choice(labels), ln)
        elif kind == 3:  # a barrier before this line
            lines.insert(i, "    bar.sync 0;")
            return "\n".join(lines) if rnd.random() < 0.5 else mutate(rnd, "\n".join(lines))
        elif kind == 4:  # another comparison
            ln = re.sub(r"setp\.(%s)\." % "|".join(CMPS), "setp.%s." % rnd.choice(CMPS), ln)
        elif kind == 5:  # another immediate
            ln = re.sub(r"(?<=[ ,+-])(\d+)(?=[;\]])", lambda m: str(rnd.choice(IMMS)), ln, count=1)
        elif kind == 6:  # the line twice
            lines.insert(i, ln)
        else:  # the line deleted
            ln = ""
        lines[i] = ln
    return "\n".join(lines)


def workload(rnd, text, params, mem_bytes=1 << 20, trace_cap=0):
    """Launch shape and inputs for a mutant: 1-3 blocks of 32-128 threads; pointer
    parameters spread over a memory image whose first half is seeded random bytes
    and second half zero; 32-bit parameters drawn from a few small values.
    `params` is [(name, offset, size)] in declaration order."""
    g = np.frombuffer(np.random.default_rng(rnd.randrange(1 << 30)).bytes(mem_bytes), np.uint8).copy()
    g[mem_bytes // 2:] = 0
    vals = []
    for j, (name, _, size) in enumerate(params):
        if size == 8:
            vals.append((name, "u64", (j * (mem_bytes // 8)) % mem_bytes))
        else:
            vals.append((name, "u32", rnd.choice([0, 1, 5, 37, 100, 256, 1000])))
    block = rnd.choice([32, 64, 96, 128])
    grid = rnd.choice([1, 2, 3])
    return Workload(name="mutant", ptx=text, grid=(grid, 1, 1), block=(block, 1, 1), params=vals, gmem=g,
                    trace_cap=trace_cap)


def launch_shape(rnd):
    """A grid of up to 6 x 3 x 2 blocks and a block of up to 64 x 4 x 2 threads (at
    most 256, any count: warps are often ragged)."""
    while True:
        block = (rnd.randint(1, 64), rnd.choice([1, 1, 2, 3, 4]), rnd.choice([1, 1, 2]))
        if block[0] * block[1] * block[2] <= 256:
            break
    grid = (rnd.randint(1, 6), rnd.choice([1, 1, 2, 3]), rnd.choice([1, 1, 2]))
    return grid, block


def latency_table(rnd, n):
    """A caller-set latency table of n classes: every entry 65535, or each drawn from
    values that include 0 and 65535."""
    if rnd.random() < 0.3:
        return [65535] * n
    return [rnd.choice([0, 1, 4, 23, 200, 300, 1000, 65535]) for _ in range(n)]
