"""Probe programs of the SASS-probe method, as simulator inputs (no simulator arithmetic).

The SASS-probe method page (teach-meaning.tistory.com/1954) measures an
instruction's latency with a loop of target instructions that either form one
dependent chain or spread over several independent accumulators, and then
controls the measurement with an empty loop (section 12.2), with chains of other
instruction kinds (section 12.3), with a sweep of the instruction count fitted to
T(N) = L * N + C (section 13), with a sweep of the accumulator count (section
14) and with a sweep of the number of warps (section 15).

Every probe here has the same loop layout as the FFMA probe of the five
workloads: the loop counter's add, half of the target instructions, the setp of
the loop condition, the other half, and the backward @p bra.  Target number k of
an iteration updates accumulator k mod n_acc.  After the loop the accumulators
are summed in order and each thread stores its sum (the page's output store that
keeps the work alive and serves as a checksum).
"""
from typing import Tuple

import numpy as np

from .configs import Workload, _align, _uniform_f32

# op -> (register type, accumulator update with {a} = accumulator, x / y = the two data registers,
#        zero literal, the add that sums the accumulators)
OPS = {
    "fma.f32": ("f32", "fma.rn.f32 {a}, %x, %y, {a};", "0f00000000", "add.f32"),
    "add.f32": ("f32", "add.f32 {a}, {a}, %x;", "0f00000000", "add.f32"),
    "mul.f32": ("f32", "mul.f32 {a}, {a}, %x;", "0f3F800000", "add.f32"),
    "add.s32": ("b32", "add.s32 {a}, {a}, %x;", "0", "add.s32"),
    "mul.s32": ("b32", "mul.lo.s32 {a}, {a}, %x;", "1", "add.s32"),
    "mad.s32": ("b32", "mad.lo.s32 {a}, %x, %y, {a};", "0", "add.s32"),
    "none": ("f32", None, "0f00000000", "add.f32"),  # the empty-loop control: no target instruction
}
OP_LATENCY_CLASS = {"fma.f32": "fp32", "add.f32": "fp32", "mul.f32": "fp32",
                    "add.s32": "int32", "mul.s32": "int32", "mad.s32": "int32", "none": None}


def chain_probe_ptx(op: str = "fma.f32", n_acc: int = 1, iters: int = 4096, per_iter: int = 32) -> str:
    """PTX of a probe: `iters` loop iterations of `per_iter` target instructions
    (op) over `n_acc` accumulators; op "none" keeps only the loop (per_iter is
    then ignored)."""
    if op not in OPS:
        raise ValueError("unknown probe op %r" % op)
    ty, upd, zero, add = OPS[op]
    assert 1 <= n_acc <= 16 and iters >= 1 and per_iter % 2 == 0
    n_targets = 0 if upd is None else per_iter
    rt = "f32" if ty == "f32" else "b32"
    L = [".version 7.5", ".target sm_80", ".address_size 64", "",
         ".visible .entry chain_probe(",
         "    .param .u64 param_x,", "    .param .u64 param_y,", "    .param .u64 param_out", ")", "{",
         "    .reg .pred %p<2>;",
         "    .reg .%s %%x;" % rt, "    .reg .%s %%y;" % rt, "    .reg .%s %%s;" % rt,
         "    .reg .%s %%acc<%d>;" % (rt, n_acc),
         "    .reg .b32 %r<6>;", "    .reg .b64 %rd<8>;", "",
         "    ld.param.u64 %rd1, [param_x];", "    ld.param.u64 %rd2, [param_y];",
         "    ld.param.u64 %rd3, [param_out];",
         "    mov.u32 %r1, %tid.x;", "    mov.u32 %r2, %ctaid.x;", "    mov.u32 %r3, %ntid.x;",
         "    mad.lo.s32 %r4, %r2, %r3, %r1;", "    mul.wide.s32 %rd4, %r4, 4;",
         "    add.s64 %rd5, %rd1, %rd4;", "    ld.global.%s %%x, [%%rd5];" % ("f32" if ty == "f32" else "u32"),
         "    add.s64 %rd6, %rd2, %rd4;", "    ld.global.%s %%y, [%%rd6];" % ("f32" if ty == "f32" else "u32")]
    acc = ["%%acc%d" % k for k in range(n_acc)]
    mov = "mov.f32" if ty == "f32" else "mov.u32"
    for a in acc:
        L.append("    %s %s, %s;" % (mov, a, zero))
    L.append("    mov.u32 %r5, 0;")
    L.append("$L__loop:")
    L.append("    add.s32 %r5, %r5, 1;")
    k = 0
    for _ in range(n_targets // 2):
        L.append("    " + upd.format(a=acc[k % n_acc]))
        k += 1
    L.append("    setp.lt.s32 %%p1, %%r5, %d;" % iters)
    for _ in range(n_targets // 2):
        L.append("    " + upd.format(a=acc[k % n_acc]))
        k += 1
    L.append("    @%p1 bra $L__loop;")
    L.append("    %s %%s, %s;" % (mov, acc[0]))
    for a in acc[1:]:
        L.append("    %s %%s, %%s, %s;" % (add, a))
    L.append("    add.s64 %rd7, %rd3, %rd4;")
    L.append("    st.global.%s [%%rd7], %%s;" % ("f32" if ty == "f32" else "u32"))
    L.append("    ret;")
    L.append("}")
    return "\n".join(L) + "\n"


def chain_probe(op: str = "fma.f32", n_acc: int = 1, iters: int = 4096, per_iter: int = 32,
                grid: int = 1, block: int = 32, seed: int = 3, trace_cap: int = 0) -> Workload:
    """A probe launch: x and y per thread (f32 uniform in [0.5, 1.5]; integer
    probes: uniform u32 words), one output word per thread."""
    nt = grid * block
    rng = np.random.default_rng(seed)
    if OPS[op][0] == "f32":
        x = _uniform_f32(rng, nt, 0.5, 1.5).view(np.uint32)
        y = _uniform_f32(rng, nt, 0.5, 1.5).view(np.uint32)
    else:
        x = rng.integers(0, 1 << 32, size=nt, dtype=np.uint32)
        y = rng.integers(0, 1 << 32, size=nt, dtype=np.uint32)
    off_x = 0
    off_y = _align(4 * nt)
    off_o = _align(off_y + 4 * nt)
    size = _align(off_o + 4 * nt)
    gmem = np.zeros(size, dtype=np.uint8)
    gmem[off_x: off_x + 4 * nt] = x.view(np.uint8)
    gmem[off_y: off_y + 4 * nt] = y.view(np.uint8)
    return Workload(
        name="probe_%s_acc%d_it%d" % (op, n_acc, iters),
        ptx=chain_probe_ptx(op, n_acc, iters, per_iter), grid=(grid, 1, 1), block=(block, 1, 1),
        params=[("param_x", "u64", off_x), ("param_y", "u64", off_y), ("param_out", "u64", off_o)],
        gmem=gmem, trace_cap=trace_cap,
        outputs={"out": (off_o, nt, "<u4")},
        meta={"op": op, "n_acc": n_acc, "iters": iters, "per_iter": 0 if op == "none" else per_iter,
              "seed": seed},
    )


# the sweeps the page runs (sections 13 to 15), as launch parameters
COUNT_SWEEP_ITERS: Tuple[int, ...] = (32, 128, 512, 2048, 4096, 8192)   # x 32 targets = 1024 ... 262144
ACC_SWEEP: Tuple[int, ...] = (1, 2, 4, 8, 16)
WARP_SWEEP: Tuple[Tuple[int, int], ...] = ((1, 1), (1, 32), (1, 64), (1, 128), (256, 128))
CONTROL_OPS: Tuple[str, ...] = ("none", "fma.f32", "add.s32", "add.f32")


# ---------------------------------------------------------------------------- pointer chase
#
# Inputs for the cache-latency model (the KernelScope page's direct-mapped L1 and L2
# in front of DRAM): a chain of dependent global loads.  Word k of the chain holds
# the byte offset of word k + 1, so every load's address comes from the previous
# load and the loads issue one after another.  Nothing here models a cache.


def chase_ptx(hops: int) -> str:
    """Each thread loads its start offset from a per-lane table, follows `hops`
    links of the chain (ld.global, then mul.wide + add.s64 to form the next
    address) and stores the last word it read."""
    assert hops >= 1
    L = [".version 7.5", ".target sm_80", ".address_size 64", "",
         ".visible .entry chase(", "    .param .u64 param_base,", "    .param .u64 param_start,",
         "    .param .u64 param_out", ")", "{",
         "    .reg .b32 %r<4>;", "    .reg .b64 %rd<8>;", "",
         "    ld.param.u64 %rd0, [param_base];", "    ld.param.u64 %rd5, [param_start];",
         "    ld.param.u64 %rd6, [param_out];",
         "    mov.u32 %r2, %tid.x;", "    mul.wide.u32 %rd3, %r2, 4;", "    add.s64 %rd4, %rd5, %rd3;",
         "    ld.global.u32 %r1, [%rd4];"]
    for _ in range(hops):
        L += ["    mul.wide.u32 %rd2, %r1, 1;", "    add.s64 %rd1, %rd0, %rd2;", "    ld.global.u32 %r1, [%rd1];"]
    L += ["    add.s64 %rd7, %rd6, %rd3;", "    st.global.u32 [%rd7], %r1;", "    ret;", "}", ""]
    return "\n".join(L)


def chase_probe(cycle, hops: int, starts=None, block: int = 32, grid: int = 1, mem_bytes: int = None,
                trace_cap: int = 64) -> Workload:
    """A chase over the byte offsets `cycle` (word at cycle[i] holds cycle[i + 1],
    the last one cycle[0]); thread %tid.x = t of every block starts at
    starts[t % len(starts)] (default: every thread at cycle[0]).  The start table
    and the output, both indexed by %tid.x, follow the chain's region on lines of
    their own."""
    cycle = [int(c) for c in cycle]
    assert all(c % 4 == 0 for c in cycle) and len(set(cycle)) == len(cycle)
    starts = [cycle[0]] if starts is None else [int(s) for s in starts]
    nthreads = block * grid
    off_start = _align(max(cycle) + 4)
    off_out = _align(off_start + 4 * nthreads)
    size = _align(off_out + 4 * nthreads) if mem_bytes is None else int(mem_bytes)
    assert size >= off_out + 4 * nthreads
    gmem = np.zeros(size, dtype=np.uint8)
    words = gmem.view("<u4")
    for i, c in enumerate(cycle):
        words[c // 4] = cycle[(i + 1) % len(cycle)]
    words[off_start // 4: off_start // 4 + nthreads] = np.array([starts[t % len(starts)] for t in range(nthreads)],
                                                                 dtype=np.uint32)
    return Workload(name="chase", ptx=chase_ptx(hops), grid=(grid, 1, 1), block=(block, 1, 1),
                    params=[("param_base", "u64", 0), ("param_start", "u64", off_start), ("param_out", "u64", off_out)],
                    gmem=gmem, trace_cap=trace_cap, outputs={"out": (off_out, nthreads, "<u4")},
                    meta={"cycle": cycle, "hops": hops, "off_start": off_start, "off_out": off_out})
