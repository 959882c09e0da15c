"""The five synthetic workloads of the simulator, as inputs.

Every workload is a PTX program in the supported subset plus a seeded initial
simulated-memory image, a parameter block, a launch shape and a trace capacity.
The programs and data shapes follow the pages' own examples:

* vector_add -- the PTX listing of the KernelScope backend documentation
  (github.com/briefgaming/kernelscope, "PTX Parser" part), with the address
  arithmetic the listing elides filled in by the plainest sequence that fits its
  register declarations (mul.wide.s32 then add.s64, no cvta).
* strided_gather -- c[i] = a[i*s] + b[i]: the strided global pattern that the
  "Memory analysis" part contrasts with the coalesced one.
* ffma_probe -- the dependent versus independent FMA chain of the SASS-probe
  method page (teach-meaning.tistory.com/1954), sections 2 and 4: 4096 outer
  iterations of 32 fma.rn.f32, one accumulator or several, result stored to
  global memory.
* bank_probe -- shared-memory stores/loads at a word stride s, the bank-conflict
  probe named in that page's section 3.
* random_stress -- seeded random programs of the subset (see randprog.py).

Inputs only: nothing here computes what the simulator computes.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

from .randprog import random_program

LAT_DEFAULT_NOTE = "default latency table: sm_80 model of the KernelScope latency page"

_PARAM_SIZES = {"u32": 4, "s32": 4, "b32": 4, "f32": 4, "u64": 8, "s64": 8, "b64": 8}


def pack_params(params: List[Tuple[str, str, int]]) -> bytes:
    """Pack (name, type, value) in declaration order, each at its natural alignment."""
    out = bytearray()
    for _name, typ, value in params:
        size = _PARAM_SIZES[typ]
        while len(out) % size:
            out.append(0)
        if typ == "f32":
            out += np.float32(value).tobytes()
        else:
            out += int(value & ((1 << (8 * size)) - 1)).to_bytes(size, "little")
    return bytes(out)


@dataclass
class Workload:
    name: str
    ptx: str
    grid: Tuple[int, int, int]
    block: Tuple[int, int, int]
    params: List[Tuple[str, str, int]]
    gmem: np.ndarray                      # uint8 initial image
    trace_cap: int
    outputs: Dict[str, Tuple[int, int, str]] = field(default_factory=dict)  # name -> (offset, count, dtype)
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def params_bytes(self) -> bytes:
        return pack_params(self.params)

    @property
    def n_blocks(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def threads_per_block(self) -> int:
        return self.block[0] * self.block[1] * self.block[2]

    @property
    def warps_per_block(self) -> int:
        return (self.threads_per_block + 31) // 32

    @property
    def n_warps(self) -> int:
        return self.n_blocks * self.warps_per_block

    def output(self, gmem: np.ndarray, name: str) -> np.ndarray:
        off, count, dt = self.outputs[name]
        return gmem[off: off + count * np.dtype(dt).itemsize].view(dt)


def _align(x: int, a: int = 4096) -> int:
    return (x + a - 1) // a * a


def _uniform_f32(rng: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    # float64 draws cast to float32
    return rng.uniform(lo, hi, size=n).astype(np.float32)


# ----------------------------------------------------------------------------- 1

VECTOR_ADD_PTX = """\
.version 7.5
.target sm_80
.address_size 64

.visible .entry vector_add(
    .param .u64 param_a,
    .param .u64 param_b,
    .param .u64 param_c,
    .param .u32 param_n
)
{
    .reg .pred %p<2>;
    .reg .f32 %f<4>;
    .reg .b32 %r<6>;
    .reg .b64 %rd<8>;

    .loc 1 2 0
    ld.param.u64 %rd1, [param_a];
    ld.param.u64 %rd2, [param_b];
    ld.param.u64 %rd3, [param_c];
    ld.param.u32 %r1, [param_n];
    mov.u32 %r2, %tid.x;
    mov.u32 %r3, %ctaid.x;
    mov.u32 %r4, %ntid.x;
    mad.lo.s32 %r5, %r3, %r4, %r2;
    setp.ge.s32 %p1, %r5, %r1;
    @%p1 bra $L__exit;
    mul.wide.s32 %rd4, %r5, 4;
    add.s64 %rd5, %rd1, %rd4;
    ld.global.f32 %f1, [%rd5];
    add.s64 %rd6, %rd2, %rd4;
    ld.global.f32 %f2, [%rd6];
    add.f32 %f3, %f1, %f2;
    add.s64 %rd7, %rd3, %rd4;
    st.global.f32 [%rd7], %f3;
$L__exit:
    ret;
}
"""


def vector_add(n: int = 1000, block: int = 256, grid: int = 4, seed: int = 0, trace_cap: int = 32) -> Workload:
    rng = np.random.default_rng(seed)
    a = _uniform_f32(rng, n, -1.0, 1.0)
    b = _uniform_f32(rng, n, -1.0, 1.0)
    off_a = 0
    off_b = _align(off_a + 4 * n)
    off_c = _align(off_b + 4 * n)
    size = _align(off_c + 4 * n, 16384)
    gmem = np.zeros(size, dtype=np.uint8)
    gmem[off_a: off_a + 4 * n] = a.view(np.uint8)
    gmem[off_b: off_b + 4 * n] = b.view(np.uint8)
    return Workload(
        name="vector_add", ptx=VECTOR_ADD_PTX, grid=(grid, 1, 1), block=(block, 1, 1),
        params=[("param_a", "u64", off_a), ("param_b", "u64", off_b), ("param_c", "u64", off_c),
                ("param_n", "u32", n)],
        gmem=gmem, trace_cap=trace_cap,
        outputs={"a": (off_a, n, "<f4"), "b": (off_b, n, "<f4"), "c": (off_c, n, "<f4")},
        meta={"n": n, "seed": seed},
    )


# ----------------------------------------------------------------------------- 2

STRIDED_PTX = """\
.version 7.5
.target sm_80
.address_size 64

.visible .entry strided_gather(
    .param .u64 param_a,
    .param .u64 param_b,
    .param .u64 param_c,
    .param .u32 param_n,
    .param .u32 param_s
)
{
    .reg .pred %p<2>;
    .reg .f32 %f<4>;
    .reg .b32 %r<8>;
    .reg .b64 %rd<9>;

    ld.param.u64 %rd1, [param_a];
    ld.param.u64 %rd2, [param_b];
    ld.param.u64 %rd3, [param_c];
    ld.param.u32 %r1, [param_n];
    ld.param.u32 %r6, [param_s];
    mov.u32 %r2, %tid.x;
    mov.u32 %r3, %ctaid.x;
    mov.u32 %r4, %ntid.x;
    mad.lo.s32 %r5, %r3, %r4, %r2;
    setp.ge.s32 %p1, %r5, %r1;
    @%p1 bra $L__exit;
    mul.lo.s32 %r7, %r5, %r6;
    mul.wide.s32 %rd4, %r7, 4;
    add.s64 %rd5, %rd1, %rd4;
    ld.global.f32 %f1, [%rd5];
    mul.wide.s32 %rd6, %r5, 4;
    add.s64 %rd7, %rd2, %rd6;
    ld.global.f32 %f2, [%rd7];
    add.f32 %f3, %f1, %f2;
    add.s64 %rd8, %rd3, %rd6;
    st.global.f32 [%rd8], %f3;
$L__exit:
    ret;
}
"""

STRIDES = (1, 2, 4, 8, 16, 32, 33)


def strided_gather(s: int, n: int = 1 << 20, block: int = 256, seed: int = None, trace_cap: int = 32) -> Workload:
    seed = s if seed is None else seed
    grid = (n + block - 1) // block
    rng = np.random.default_rng(seed)
    a = _uniform_f32(rng, n * s, -1.0, 1.0)
    b = _uniform_f32(rng, n, -1.0, 1.0)
    off_a = 0
    off_b = _align(off_a + 4 * n * s)
    off_c = _align(off_b + 4 * n)
    size = _align(off_c + 4 * n)
    gmem = np.zeros(size, dtype=np.uint8)
    gmem[off_a: off_a + 4 * n * s] = a.view(np.uint8)
    gmem[off_b: off_b + 4 * n] = b.view(np.uint8)
    return Workload(
        name="strided_gather_s%d" % s, ptx=STRIDED_PTX, grid=(grid, 1, 1), block=(block, 1, 1),
        params=[("param_a", "u64", off_a), ("param_b", "u64", off_b), ("param_c", "u64", off_c),
                ("param_n", "u32", n), ("param_s", "u32", s)],
        gmem=gmem, trace_cap=trace_cap,
        outputs={"a": (off_a, n * s, "<f4"), "b": (off_b, n, "<f4"), "c": (off_c, n, "<f4")},
        meta={"s": s, "n": n, "seed": seed},
    )


# ----------------------------------------------------------------------------- 3

def ffma_probe_ptx(n_acc: int = 1, iters: int = 4096, fma_per_half: int = 16) -> str:
    """The FMA latency probe: per thread `iters` iterations of 2 * fma_per_half
    fma.rn.f32; FMA number k of an iteration updates accumulator k mod n_acc, so
    n_acc = 1 is the dependent chain and n_acc = 8 the independent variant.
    Loop layout: add (counter) -> half the FMAs -> setp -> other half -> @p bra."""
    assert 1 <= n_acc <= 16
    L = [".version 7.5", ".target sm_80", ".address_size 64", "",
         ".visible .entry ffma_probe(",
         "    .param .u64 param_x,", "    .param .u64 param_y,", "    .param .u64 param_out", ")", "{",
         "    .reg .pred %p<2>;", "    .reg .f32 %%f<%d>;" % (3 + n_acc + 1), "    .reg .b32 %r<6>;",
         "    .reg .b64 %rd<8>;", "",
         "    ld.param.u64 %rd1, [param_x];", "    ld.param.u64 %rd2, [param_y];",
         "    ld.param.u64 %rd3, [param_out];",
         "    mov.u32 %r1, %tid.x;", "    mov.u32 %r2, %ctaid.x;", "    mov.u32 %r3, %ntid.x;",
         "    mad.lo.s32 %r4, %r2, %r3, %r1;", "    mul.wide.s32 %rd4, %r4, 4;",
         "    add.s64 %rd5, %rd1, %rd4;", "    ld.global.f32 %f1, [%rd5];",
         "    add.s64 %rd6, %rd2, %rd4;", "    ld.global.f32 %f2, [%rd6];"]
    acc = ["%%f%d" % (3 + k) for k in range(n_acc)]
    for a in acc:
        L.append("    mov.f32 %s, 0f00000000;" % a)
    L.append("    mov.u32 %r5, 0;")
    L.append("$L__loop:")
    L.append("    add.s32 %r5, %r5, 1;")
    k = 0
    for _ in range(fma_per_half):
        L.append("    fma.rn.f32 {0}, %f1, %f2, {0};".format(acc[k % n_acc]))
        k += 1
    L.append("    setp.lt.s32 %%p1, %%r5, %d;" % iters)
    for _ in range(fma_per_half):
        L.append("    fma.rn.f32 {0}, %f1, %f2, {0};".format(acc[k % n_acc]))
        k += 1
    L.append("    @%p1 bra $L__loop;")
    s = acc[0]
    if n_acc > 1:
        s = "%%f%d" % (3 + n_acc)
        L.append("    add.f32 %s, %s, %s;" % (s, acc[0], acc[1]))
        for a in acc[2:]:
            L.append("    add.f32 %s, %s, %s;" % (s, s, a))
    L.append("    add.s64 %rd7, %rd3, %rd4;")
    L.append("    st.global.f32 [%%rd7], %s;" % s)
    L.append("    ret;")
    L.append("}")
    return "\n".join(L) + "\n"


def ffma_probe(n_acc: int = 1, iters: int = 4096, grid: int = 1024, block: int = 256, seed: int = 3,
               trace_cap: int = 4096, fma_per_half: int = 16) -> Workload:
    nt = grid * block
    rng = np.random.default_rng(seed)
    x = _uniform_f32(rng, nt, 0.5, 1.5)
    y = _uniform_f32(rng, nt, 0.5, 1.5)
    off_x = 0
    off_y = _align(4 * nt)
    off_o = _align(off_y + 4 * nt)
    size = _align(off_o + 4 * nt)
    gmem = np.zeros(size, dtype=np.uint8)
    gmem[off_x: off_x + 4 * nt] = x.view(np.uint8)
    gmem[off_y: off_y + 4 * nt] = y.view(np.uint8)
    return Workload(
        name="ffma_probe_acc%d" % n_acc, ptx=ffma_probe_ptx(n_acc, iters, fma_per_half),
        grid=(grid, 1, 1), block=(block, 1, 1),
        params=[("param_x", "u64", off_x), ("param_y", "u64", off_y), ("param_out", "u64", off_o)],
        gmem=gmem, trace_cap=trace_cap,
        outputs={"x": (off_x, nt, "<f4"), "y": (off_y, nt, "<f4"), "out": (off_o, nt, "<f4")},
        meta={"n_acc": n_acc, "iters": iters, "fma_per_iter": 2 * fma_per_half, "seed": seed},
    )


# ----------------------------------------------------------------------------- 4

def bank_probe_ptx(iters: int = 1024, shared_bytes: int = 32768) -> str:
    """Per thread: w = laneid * s; x = v[w]; then `iters` times {st.shared [4w], x;
    bar.sync 0; ld.shared y, [4w]; acc += y}; finally out[gtid] = acc."""
    return """\
.version 7.5
.target sm_80
.address_size 64

.visible .entry bank_probe(
    .param .u64 param_v,
    .param .u64 param_out,
    .param .u32 param_s
)
{
    .reg .pred %%p<2>;
    .reg .b32 %%r<14>;
    .reg .b64 %%rd<7>;
    .shared .align 4 .b8 smem[%d];

    ld.param.u64 %%rd1, [param_v];
    ld.param.u64 %%rd2, [param_out];
    ld.param.u32 %%r1, [param_s];
    mov.u32 %%r2, %%laneid;
    mul.lo.s32 %%r3, %%r2, %%r1;
    mul.wide.s32 %%rd3, %%r3, 4;
    add.s64 %%rd4, %%rd1, %%rd3;
    ld.global.f32 %%r9, [%%rd4];
    mov.u32 %%r4, smem;
    mul.lo.s32 %%r5, %%r3, 4;
    add.s32 %%r6, %%r4, %%r5;
    mov.u32 %%r7, 0;
    mov.u32 %%r8, 0;
$L__loop:
    st.shared.f32 [%%r6], %%r9;
    bar.sync 0;
    ld.shared.f32 %%r10, [%%r6];
    add.s32 %%r7, %%r7, %%r10;
    add.s32 %%r8, %%r8, 1;
    setp.lt.s32 %%p1, %%r8, %d;
    @%%p1 bra $L__loop;
    mov.u32 %%r11, %%tid.x;
    mov.u32 %%r12, %%ctaid.x;
    mov.u32 %%r13, %%ntid.x;
    mad.lo.s32 %%r11, %%r12, %%r13, %%r11;
    mul.wide.s32 %%rd5, %%r11, 4;
    add.s64 %%rd6, %%rd2, %%rd5;
    st.global.u32 [%%rd6], %%r7;
    ret;
}
""" % (shared_bytes, iters)


def bank_probe(s: int, iters: int = 1024, grid: int = 256, block: int = 1024, seed: int = 4,
               trace_cap: int = 256) -> Workload:
    nt = grid * block
    rng = np.random.default_rng(seed)
    v = rng.integers(-(1 << 31), 1 << 31, size=8192, dtype=np.int32)
    off_v = 0
    off_o = _align(4 * 8192)
    size = _align(off_o + 4 * nt)
    gmem = np.zeros(size, dtype=np.uint8)
    gmem[off_v: off_v + 4 * 8192] = v.view(np.uint8)
    return Workload(
        name="bank_probe_s%d" % s, ptx=bank_probe_ptx(iters), grid=(grid, 1, 1), block=(block, 1, 1),
        params=[("param_v", "u64", off_v), ("param_out", "u64", off_o), ("param_s", "u32", s)],
        gmem=gmem, trace_cap=trace_cap,
        outputs={"v": (off_v, 8192, "<i4"), "out": (off_o, nt, "<u4")},
        meta={"s": s, "iters": iters, "seed": seed},
    )


# ----------------------------------------------------------------------------- 5

def random_stress(prog_seed: int = 0, grid: int = 65536, block: int = 256, mem_seed: int = 5,
                  gmem_bytes: int = 1 << 30, n_instr: int = 2000, trace_cap: int = 2048) -> Workload:
    """Seeded random program of the subset over a `gmem_bytes` image of uniform
    random 32-bit words.  Memory map: reads from R = [0, gmem/2); thread-private
    writes to W1 = [gmem/2, 3 gmem/4) and W4 = [3 gmem/4, gmem)."""
    nt = grid * block
    assert gmem_bytes % 4 == 0
    r_base, w1_base, w4_base = 0, gmem_bytes // 2, gmem_bytes // 2 + gmem_bytes // 4
    ptx, meta = random_program(prog_seed, n_instr=n_instr, n_threads=nt, r_bytes=gmem_bytes // 2,
                               w1_bytes=gmem_bytes // 4, w4_bytes=gmem_bytes // 4)
    rng = np.random.default_rng(mem_seed)
    words = rng.integers(0, 1 << 32, size=gmem_bytes // 4, dtype=np.uint32)
    gmem = words.view(np.uint8)
    meta.update({"prog_seed": prog_seed, "mem_seed": mem_seed})
    return Workload(
        name="random_stress_p%d" % prog_seed, ptx=ptx, grid=(grid, 1, 1), block=(block, 1, 1),
        params=[("param_r", "u64", r_base), ("param_w1", "u64", w1_base), ("param_w4", "u64", w4_base)],
        gmem=gmem, trace_cap=trace_cap,
        outputs={"w1": (w1_base, gmem_bytes // 16, "<u4"), "w4": (w4_base, gmem_bytes // 16, "<u4")},
        meta=meta,
    )
