"""Small seeded test programs and inputs (inputs only, no simulator arithmetic).

These exercise single features: f32 arithmetic on edge operands, straight-line
FMA chains, worst-case divergence nesting, arbitrary per-lane address patterns
for the memory analyser, and small control-flow shapes.
"""
import numpy as np

from .configs import Workload, _align

HEADER = ".version 7.5\n.target sm_80\n.address_size 64\n\n"

F32_EDGE = [0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x807FFFFF, 0x00800000,
            0x80800000, 0x3F800000, 0xBF800000, 0x3F800001, 0x3F7FFFFF, 0x7F7FFFFF, 0xFF7FFFFF,
            0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x7F800001, 0x34000000, 0x33800000,
            0x4B800000, 0x4B7FFFFF, 0x3EAAAAAB, 0x40490FDB, 0x00400000, 0x0C000000, 0x4C000000,
            0x5F000000, 0x1F000000, 0x7F000000, 0x01000000]


def f32_operands(n: int, seed: int = 11) -> np.ndarray:
    """(n, 3) uint32 operand bit patterns: edge values crossed with each other,
    then random patterns with every exponent represented, then near-cancelling
    and near-overflow/underflow pairs."""
    rng = np.random.default_rng(seed)
    rows = []
    E = np.array(F32_EDGE, dtype=np.uint32)
    for a in E:
        for b in E:
            rows.append((a, b, E[(int(a) ^ int(b)) % len(E)]))
    out = np.array(rows, dtype=np.uint32)
    k = max(0, n - len(out))
    rnd = rng.integers(0, 1 << 32, size=(k, 3), dtype=np.uint32)
    # a quarter: exponents near each other (cancellation, close magnitudes)
    q = k // 4
    if q:
        a = rnd[:q, 0]
        b = (a ^ rng.integers(0, 1 << 8, size=q, dtype=np.uint32)) ^ np.uint32(0x80000000)
        rnd[:q, 1] = b
        # addend close to -(a*b)'s magnitude range
        rnd[:q, 2] = (rnd[:q, 2] & np.uint32(0x807FFFFF)) | (((a >> 23) & 0xFF) << 23).astype(np.uint32)
    # a quarter: small exponents (subnormal results)
    if q:
        rnd[q:2 * q, :] &= np.uint32(0x83FFFFFF)
    out = np.concatenate([out, rnd])[:max(n, len(out))]
    return out


F32_OPS_PTX = HEADER + """\
.visible .entry f32_ops(
    .param .u64 param_in,
    .param .u64 param_out,
    .param .u32 param_n
)
{
    .reg .pred %p<2>;
    .reg .b32 %r<16>;
    .reg .b64 %rd<8>;

    ld.param.u64 %rd1, [param_in];
    ld.param.u64 %rd2, [param_out];
    ld.param.u32 %r1, [param_n];
    mov.u32 %r2, %tid.x;
    mov.u32 %r3, %ctaid.x;
    mov.u32 %r4, %ntid.x;
    mad.lo.s32 %r5, %r3, %r4, %r2;
    setp.ge.u32 %p1, %r5, %r1;
    @%p1 bra $L__exit;
    mul.wide.u32 %rd3, %r5, 12;
    add.s64 %rd4, %rd1, %rd3;
    ld.global.f32 %r6, [%rd4];
    ld.global.f32 %r7, [%rd4+4];
    ld.global.f32 %r8, [%rd4+8];
    add.f32 %r9, %r6, %r7;
    sub.f32 %r10, %r6, %r7;
    mul.f32 %r11, %r6, %r7;
    fma.rn.f32 %r12, %r6, %r7, %r8;
    mul.wide.u32 %rd5, %r5, 16;
    add.s64 %rd6, %rd2, %rd5;
    st.global.f32 [%rd6], %r9;
    st.global.f32 [%rd6+4], %r10;
    st.global.f32 [%rd6+8], %r11;
    st.global.f32 [%rd6+12], %r12;
$L__exit:
    ret;
}
"""


def f32_ops(n: int = 8192, block: int = 256, seed: int = 11) -> Workload:
    ops = f32_operands(n, seed)
    n = len(ops)
    off_in = 0
    off_out = _align(12 * n)
    size = _align(off_out + 16 * n)
    gmem = np.zeros(size, dtype=np.uint8)
    gmem[: 12 * n] = ops.reshape(-1).view(np.uint8)
    grid = (n + block - 1) // block
    return Workload(name="f32_ops", ptx=F32_OPS_PTX, grid=(grid, 1, 1), block=(block, 1, 1),
                    params=[("param_in", "u64", off_in), ("param_out", "u64", off_out), ("param_n", "u32", n)],
                    gmem=gmem, trace_cap=32,
                    outputs={"in": (off_in, 3 * n, "<u4"), "out": (off_out, 4 * n, "<u4")}, meta={"n": n})


def fma_chain_ptx(n_fma: int, n_acc: int) -> str:
    """Straight-line chain: n_fma fma.rn.f32 cycling over n_acc accumulators, then
    a store of accumulator 0 (which depends on the last FMA into it)."""
    L = [HEADER + ".visible .entry fma_chain(\n    .param .u64 param_out\n)\n{",
         "    .reg .f32 %%f<%d>;" % (2 + n_acc), "    .reg .b64 %rd<2>;",
         "    ld.param.u64 %rd1, [param_out];",
         "    mov.f32 %f0, 0f3F800000;", "    mov.f32 %f1, 0f3F000000;"]
    for k in range(n_fma):
        a = "%%f%d" % (2 + k % n_acc)
        L.append("    fma.rn.f32 %s, %%f0, %%f1, %s;" % (a, a))
    last = "%%f%d" % (2 + (n_fma - 1) % n_acc)
    L.append("    st.global.f32 [%%rd1], %s;" % last)
    L.append("    ret;\n}\n")
    return "\n".join(L)


def staircase_ptx(levels: int = 31) -> str:
    """Worst-case divergence nesting: at level k lane k leaves on an if/else whose
    taken side jumps to its own block; every split adds two stack entries."""
    L = [HEADER + ".visible .entry staircase(\n    .param .u64 param_out\n)\n{",
         "    .reg .pred %p<2>;", "    .reg .b32 %r<4>;", "    .reg .b64 %rd<4>;",
         "    ld.param.u64 %rd1, [param_out];", "    mov.u32 %r1, %laneid;", "    mov.u32 %r2, 0;"]
    # S_k = setp_k; @p bra t_k; S_{k+1}; bra e_k; t_k: r2 += k+1; e_k: r2 += 1
    for k in range(levels):
        L.append("    setp.eq.u32 %%p1, %%r1, %d;" % k)
        L.append("    @%%p1 bra $L__t%d;" % k)
    L.append("    add.s32 %r2, %r2, 1000;")
    for k in range(levels - 1, -1, -1):
        L.append("    bra.uni $L__e%d;" % k)
        L.append("$L__t%d:" % k)
        L.append("    add.s32 %%r2, %%r2, %d;" % (k + 1))
        L.append("$L__e%d:" % k)
        L.append("    add.s32 %r2, %r2, 1;")
    L.append("    mul.wide.u32 %rd2, %r1, 4;")
    L.append("    add.s64 %rd3, %rd1, %rd2;")
    L.append("    st.global.u32 [%rd3], %r2;")
    L.append("    ret;\n}\n")
    return "\n".join(L)


ADDR_PROBE_PTX = HEADER + """\
.visible .entry addr_probe(
    .param .u64 param_gaddr,
    .param .u64 param_saddr,
    .param .u64 param_guard,
    .param .u64 param_out
)
{
    .reg .pred %p<3>;
    .reg .b32 %r<12>;
    .reg .b64 %rd<12>;
    .shared .align 8 .b8 win[4096];

    ld.param.u64 %rd1, [param_gaddr];
    ld.param.u64 %rd2, [param_guard];
    ld.param.u64 %rd3, [param_out];
    ld.param.u64 %rd10, [param_saddr];
    mov.u32 %r2, %tid.x;
    mov.u32 %r3, %ctaid.x;
    mov.u32 %r4, %ntid.x;
    mad.lo.s32 %r5, %r3, %r4, %r2;
    mul.wide.u32 %rd4, %r5, 8;
    add.s64 %rd5, %rd1, %rd4;
    ld.global.u64 %rd6, [%rd5];
    mul.wide.u32 %rd7, %r5, 4;
    add.s64 %rd8, %rd2, %rd7;
    ld.global.u32 %r6, [%rd8];
    add.s64 %rd11, %rd10, %rd7;
    ld.global.u32 %r8, [%rd11];
    setp.ne.u32 %p1, %r6, 0;
    mov.u32 %r7, 0;
    @%p1 ld.global.u32 %r7, [%rd6];
    @%p1 st.global.u32 [%rd6], %r7;
    @%p1 ld.shared.u32 %r9, [%r8];
    @%p1 st.shared.u32 [%r8], %r9;
    add.s64 %rd9, %rd3, %rd7;
    st.global.u32 [%rd9], %r7;
    ret;
}
"""


def addr_probe(gaddr: np.ndarray, saddr: np.ndarray, guard: np.ndarray, data_bytes: int,
               block: int = 256, seed: int = 12) -> Workload:
    """One warp per address vector: lane l of warp w loads/stores global address
    gaddr[32 w + l] (a byte offset into the data region at 0) and shared address
    saddr[32 w + l] when guard[32 w + l] != 0.  Stores write back what was loaded,
    so repeated or shared addresses are benign."""
    n = len(gaddr)
    assert n % block == 0 and len(saddr) == n and len(guard) == n
    rng = np.random.default_rng(seed)
    off_data = 0
    off_g = _align(data_bytes)
    off_s = _align(off_g + 8 * n)
    off_guard = _align(off_s + 4 * n)
    off_out = _align(off_guard + 4 * n)
    size = _align(off_out + 4 * n)
    gmem = np.zeros(size, dtype=np.uint8)
    gmem[:data_bytes] = rng.integers(0, 256, size=data_bytes, dtype=np.uint8)
    gmem[off_g: off_g + 8 * n] = np.asarray(gaddr, dtype=np.uint64).view(np.uint8)
    gmem[off_s: off_s + 4 * n] = np.asarray(saddr, dtype=np.uint32).view(np.uint8)
    gmem[off_guard: off_guard + 4 * n] = np.asarray(guard, dtype=np.uint32).view(np.uint8)
    return Workload(name="addr_probe", ptx=ADDR_PROBE_PTX, grid=(n // block, 1, 1), block=(block, 1, 1),
                    params=[("param_gaddr", "u64", off_g), ("param_saddr", "u64", off_s),
                            ("param_guard", "u64", off_guard), ("param_out", "u64", off_out)],
                    gmem=gmem, trace_cap=32, outputs={"out": (off_out, n, "<u4")}, meta={"n": n})


def random_cfg_ptx(seed: int, n_instr: int = 24, loops: bool = False, with_ret: bool = True) -> str:
    """A small random control-flow shape over lanes: guards come from per-lane
    data (lane id bits and loaded words), branches go forward (or also backward
    when `loops`, for post-dominator checks only, never executed), predicated
    ret may appear.  Every instruction body is an add into a per-lane checksum
    register so executions are observable in memory."""
    rng = np.random.default_rng(seed)
    L = [HEADER + ".visible .entry cfg(\n    .param .u64 param_in,\n    .param .u64 param_out\n)\n{",
         "    .reg .pred %p<4>;", "    .reg .b32 %r<8>;", "    .reg .b64 %rd<6>;",
         "    ld.param.u64 %rd1, [param_in];", "    ld.param.u64 %rd2, [param_out];",
         "    mov.u32 %r1, %tid.x;", "    mov.u32 %r2, %ctaid.x;", "    mov.u32 %r3, %ntid.x;",
         "    mad.lo.s32 %r4, %r2, %r3, %r1;", "    mul.wide.u32 %rd3, %r4, 4;",
         "    add.s64 %rd4, %rd1, %rd3;", "    ld.global.u32 %r5, [%rd4];", "    mov.u32 %r6, 0;",
         "    setp.ne.u32 %p0, %r5, 0;", "    setp.lt.u32 %p1, %r5, 1000;",
         "    setp.gt.u32 %p2, %r5, 2000;", "    setp.eq.u32 %p3, %r1, 0;"]
    base = len(L) - 5  # number of instructions so far (the header and .reg lines are not instructions)
    body = []
    for i in range(n_instr):
        r = rng.random()
        if r < 0.35:
            lo = i + 2 if not loops or rng.random() < 0.7 else 0
            hi = n_instr + 1
            tgt = int(rng.integers(lo, hi)) if lo < hi else n_instr
            neg = "!" if rng.random() < 0.5 else ""
            body.append(("bra", "@%s%%p%d bra $L__b%d;" % (neg, int(rng.integers(0, 4)), tgt), tgt))
        elif r < 0.42 and with_ret:
            body.append(("ret", "@%%p%d ret;" % int(rng.integers(0, 4)), None))
        elif r < 0.5:
            body.append(("flip", "setp.lt.u32 %%p%d, %%r5, %d;" % (int(rng.integers(0, 4)),
                                                                   int(rng.integers(0, 3000))), None))
        else:
            body.append(("add", "add.s32 %%r6, %%r6, %d;" % (1 << (i % 24)), None))
    targets = {t for k, _, t in body if k == "bra"}
    for i, (_, text, _) in enumerate(body):
        if i in targets:
            L.append("$L__b%d:" % i)
        L.append("    " + text)
    if n_instr in targets:
        L.append("$L__b%d:" % n_instr)
    L += ["    add.s64 %rd5, %rd2, %rd3;", "    st.global.u32 [%rd5], %r6;", "    ret;", "}"]
    return "\n".join(L) + "\n"


def shared_edges_ptx() -> str:
    """The largest shared window (65536 bytes) at its edges, on 256-thread blocks.
    Thread t stores t + 1 at word t and t + 7 at word 16128 + t (the last KiB),
    then, after a barrier, loads its neighbour's two words (neighbour t + 1, or 0
    for t = 255), the window's last word, one word past the end and a misaligned
    word (both fault and read 0), and the last 8 bytes as one 64-bit load.  The
    results go to out[32 t + 0, 4, 8, 12, 16] (u32) and out[32 t + 24] (u64)."""
    return HEADER + """\
.visible .entry shared_edges(
    .param .u64 param_out
)
{
    .reg .pred %p<2>;
    .reg .b32 %r<20>;
    .reg .b64 %rd<6>;
    .shared .align 8 .b8 smem[65536];

    ld.param.u64 %rd1, [param_out];
    mov.u32 %r1, %tid.x;
    mov.u32 %r2, smem;
    mul.lo.s32 %r3, %r1, 4;
    add.s32 %r4, %r2, %r3;
    add.s32 %r5, %r4, 64512;
    add.s32 %r6, %r1, 1;
    add.s32 %r7, %r1, 7;
    st.shared.u32 [%r4], %r6;
    st.shared.u32 [%r5], %r7;
    bar.sync 0;
    setp.eq.u32 %p1, %r1, 255;
    add.s32 %r8, %r1, 1;
    mov.u32 %r9, 0;
    selp.b32 %r8, %r9, %r8, %p1;
    mul.lo.s32 %r10, %r8, 4;
    add.s32 %r11, %r2, %r10;
    ld.shared.u32 %r12, [%r11];
    add.s32 %r13, %r11, 64512;
    ld.shared.u32 %r14, [%r13];
    ld.shared.u32 %r15, [%r2+65532];
    ld.shared.u32 %r16, [%r2+65536];
    ld.shared.u32 %r17, [%r2+2];
    ld.shared.u64 %rd2, [%r2+65528];
    mov.u32 %r18, %ctaid.x;
    mov.u32 %r19, %ntid.x;
    mad.lo.s32 %r18, %r18, %r19, %r1;
    mul.wide.u32 %rd3, %r18, 32;
    add.s64 %rd4, %rd1, %rd3;
    st.global.u32 [%rd4], %r12;
    st.global.u32 [%rd4+4], %r14;
    st.global.u32 [%rd4+8], %r15;
    st.global.u32 [%rd4+12], %r16;
    st.global.u32 [%rd4+16], %r17;
    st.global.u64 [%rd4+24], %rd2;
    ret;
}
"""


# Producer/consumer pairs of latency_classes_ptx: (producer, latency class of the
# producer, consumer reading the producer's destination).
LATENCY_PAIRS = [
    ("add.s32 %r3, %r1, %r2;", "int32", "add.s32 %r11, %r3, 0;"),
    ("sub.s32 %r3, %r1, %r2;", "int32", "add.s32 %r11, %r3, 0;"),
    ("mul.lo.s32 %r3, %r1, %r2;", "int32", "add.s32 %r11, %r3, 0;"),
    ("mad.lo.s32 %r3, %r1, %r2, %r1;", "int32", "add.s32 %r11, %r3, 0;"),
    ("add.s64 %rd2, %rd1, %rd1;", "int64", "add.s64 %rd10, %rd2, 0;"),
    ("sub.s64 %rd2, %rd1, %rd1;", "int64", "add.s64 %rd10, %rd2, 0;"),
    ("mul.lo.s64 %rd2, %rd1, %rd1;", "int64", "add.s64 %rd10, %rd2, 0;"),
    ("mad.lo.s64 %rd2, %rd1, %rd1, %rd1;", "int64", "add.s64 %rd10, %rd2, 0;"),
    ("mul.wide.s32 %rd2, %r1, %r2;", "int32", "add.s64 %rd10, %rd2, 0;"),  # 32-bit operands
    ("mul.wide.u32 %rd2, %r1, %r2;", "int32", "add.s64 %rd10, %rd2, 0;"),
    ("add.f32 %f2, %f1, %f1;", "fp32", "add.f32 %f10, %f2, %f2;"),
    ("sub.f32 %f2, %f1, %f1;", "fp32", "add.f32 %f10, %f2, %f2;"),
    ("mul.f32 %f2, %f1, %f1;", "fp32", "add.f32 %f10, %f2, %f2;"),
    ("fma.rn.f32 %f2, %f1, %f1, %f1;", "fp32", "add.f32 %f10, %f2, %f2;"),
    ("setp.lt.s32 %p1, %r1, %r2;", "setp", "selp.b32 %r12, %r1, %r2, %p1;"),
    ("setp.gt.f32 %p1, %f1, %f1;", "setp", "selp.b32 %r12, %r1, %r2, %p1;"),
    ("setp.eq.u64 %p1, %rd1, %rd1;", "setp", "selp.b32 %r12, %r1, %r2, %p1;"),
    ("selp.b32 %r3, %r1, %r2, %p1;", "selp", "add.s32 %r11, %r3, 0;"),
    ("mov.u32 %r3, %r1;", "mov", "add.s32 %r11, %r3, 0;"),
    ("mov.u32 %r3, 12345;", "mov", "add.s32 %r11, %r3, 0;"),
    ("mov.u32 %r3, %tid.x;", "mov", "add.s32 %r11, %r3, 0;"),
    ("mov.u32 %r4, sm;", "mov", "add.s32 %r11, %r4, 0;"),
    ("ld.param.u32 %r3, [param_q];", "ld_param", "add.s32 %r11, %r3, 0;"),
    ("ld.global.u32 %r3, [%rd1];", "ld_global", "add.s32 %r11, %r3, 0;"),
    ("ld.global.u64 %rd2, [%rd1];", "ld_global", "add.s64 %rd10, %rd2, 0;"),
    ("ld.shared.u32 %r3, [%r4];", "ld_shared", "add.s32 %r11, %r3, 0;"),
    # the issue rule's sources: a guard, a store's value and address, a load's address
    ("setp.lt.s32 %p1, %r1, %r2;", "setp", "@%p1 add.s32 %r11, %r1, 0;"),
    ("add.s32 %r3, %r1, %r2;", "int32", "st.shared.u32 [%r4], %r3;"),
    ("mov.u32 %r5, sm;", "mov", "st.shared.u32 [%r5], %r1;"),
    ("add.s64 %rd3, %rd1, 0;", "int64", "ld.global.u32 %r11, [%rd3];"),
    # an instruction no lane passes the guard of still sets its destination's ready cycle
    ("@%p0 add.s32 %r3, %r1, %r2;", "int32", "add.s32 %r11, %r3, 0;"),
]


def latency_classes_ptx() -> str:
    """A prologue that makes the pairs' sources ready (each followed by a consumer;
    %p0 is false and %p1 true), then LATENCY_PAIRS in order, then ret.  Every producer reads only registers
    whose values are long ready, and every consumer reads its producer's result."""
    pro = ["ld.param.u64 %rd1, [param_p];", "add.s64 %rd9, %rd1, 0;",
           "mov.u32 %r1, 7;", "add.s32 %r9, %r1, 0;",
           "mov.u32 %r2, 3;", "add.s32 %r9, %r2, 0;",
           "mov.f32 %f1, 0f3F800000;", "add.f32 %f9, %f1, %f1;",
           "setp.ne.s32 %p1, %r1, %r2;", "selp.b32 %r9, %r1, %r2, %p1;",
           "setp.eq.s32 %p0, %r1, %r2;", "selp.b32 %r9, %r1, %r2, %p0;"]
    body = [x for p, _, c in LATENCY_PAIRS for x in (p, c)]
    return HEADER + (".visible .entry latency_classes(\n    .param .u64 param_p,\n    .param .u32 param_q\n)\n{\n"
                     "    .reg .pred %p<2>;\n    .reg .b32 %r<13>;\n    .reg .b64 %rd<11>;\n    .reg .f32 %f<11>;\n"
                     "    .shared .align 8 .b8 sm[64];\n") + "".join("    %s\n" % x for x in pro + body + ["ret;"]) + "}\n"


def block_reduce_ptx(block: int = 256) -> str:
    """A shared-memory tree reduction of u32 words over `block` (a power of two)
    threads: thread t loads in[gid] into sm[t]; then, for s = block/2 .. 1, the
    threads t < s add sm[t + s] into sm[t] behind a branch (divergent once s < 32)
    and every thread meets at a bar.sync; thread 0 stores sm[0] to out[blockid].
    The steps are unrolled (the subset has no shifts)."""
    assert block & (block - 1) == 0 and 2 <= block <= 1024
    L = [HEADER + ".visible .entry block_reduce(\n    .param .u64 param_in,\n    .param .u64 param_out\n)\n{",
         "    .reg .pred %p<2>;", "    .reg .b32 %r<12>;", "    .reg .b64 %rd<8>;",
         "    .shared .align 4 .b8 sm[%d];" % (4 * block),
         "    ld.param.u64 %rd1, [param_in];", "    ld.param.u64 %rd2, [param_out];",
         "    mov.u32 %r1, %tid.x;", "    mov.u32 %r2, %ctaid.x;", "    mov.u32 %r3, %ntid.x;",
         "    mad.lo.s32 %r4, %r2, %r3, %r1;", "    mul.wide.u32 %rd3, %r4, 4;", "    add.s64 %rd4, %rd1, %rd3;",
         "    ld.global.u32 %r5, [%rd4];", "    mov.u32 %r6, sm;", "    mul.lo.s32 %r7, %r1, 4;",
         "    add.s32 %r8, %r6, %r7;", "    st.shared.u32 [%r8], %r5;", "    bar.sync 0;"]
    s, k = block // 2, 0
    while s >= 1:
        L += ["    setp.ge.u32 %%p1, %%r1, %d;" % s, "    @%%p1 bra $L__s%d;" % k,
              "    ld.shared.u32 %%r9, [%%r8+%d];" % (4 * s), "    ld.shared.u32 %r10, [%r8];",
              "    add.s32 %r10, %r10, %r9;", "    st.shared.u32 [%r8], %r10;",
              "$L__s%d:" % k, "    bar.sync 0;"]
        s //= 2
        k += 1
    L += ["    setp.ne.u32 %p1, %r1, 0;", "    @%p1 bra $L__end;", "    ld.shared.u32 %r11, [%r6];",
          "    mul.wide.u32 %rd5, %r2, 4;", "    add.s64 %rd6, %rd2, %rd5;", "    st.global.u32 [%rd6], %r11;",
          "$L__end:", "    ret;", "}"]
    return "\n".join(L) + "\n"


def tile_transpose_ptx(pad: int = 0) -> str:
    """out = in transposed, for an n x n u32 matrix (n = 32 * grid.x, grid square)
    through a 32 x (32 + pad) shared tile, on 32 x 32 blocks: thread (x, y) of block
    (bx, by) stores in[32 by + y][32 bx + x] at tile[y][x] (a row: stride 1), meets
    the others at a bar.sync, and writes tile[x][y] (a column: stride 32 + pad
    words, so 32-way bank conflicts when pad = 0, none when pad = 1) to
    out[32 bx + y][32 by + x]."""
    row = 32 + pad
    return HEADER + """\
.visible .entry tile_transpose(
    .param .u64 param_in,
    .param .u64 param_out
)
{
    .reg .b32 %%r<20>;
    .reg .b64 %%rd<8>;
    .shared .align 4 .b8 tile[%d];

    ld.param.u64 %%rd1, [param_in];
    ld.param.u64 %%rd2, [param_out];
    mov.u32 %%r1, %%tid.x;
    mov.u32 %%r2, %%tid.y;
    mov.u32 %%r3, %%ctaid.x;
    mov.u32 %%r4, %%ctaid.y;
    mov.u32 %%r5, %%nctaid.x;
    mul.lo.s32 %%r6, %%r5, 32;
    mad.lo.s32 %%r7, %%r4, 32, %%r2;
    mad.lo.s32 %%r8, %%r3, 32, %%r1;
    mad.lo.s32 %%r9, %%r7, %%r6, %%r8;
    mul.wide.u32 %%rd3, %%r9, 4;
    add.s64 %%rd4, %%rd1, %%rd3;
    ld.global.u32 %%r10, [%%rd4];
    mov.u32 %%r11, tile;
    mad.lo.s32 %%r12, %%r2, %d, %%r1;
    mad.lo.s32 %%r13, %%r12, 4, %%r11;
    st.shared.u32 [%%r13], %%r10;
    bar.sync 0;
    mad.lo.s32 %%r14, %%r1, %d, %%r2;
    mad.lo.s32 %%r15, %%r14, 4, %%r11;
    ld.shared.u32 %%r16, [%%r15];
    mad.lo.s32 %%r17, %%r3, 32, %%r2;
    mad.lo.s32 %%r18, %%r4, 32, %%r1;
    mad.lo.s32 %%r19, %%r17, %%r6, %%r18;
    mul.wide.u32 %%rd5, %%r19, 4;
    add.s64 %%rd6, %%rd2, %%rd5;
    st.global.u32 [%%rd6], %%r16;
    ret;
}
""" % (4 * 32 * row, row, row)


def stencil3_ptx() -> str:
    """out[i] = in[i-1] + in[i] + in[i+1] (u32, wrapping) for 0 < i < n-1 and
    out[i] = in[i] at the two ends, one thread per i (threads at i >= n do
    nothing).  The boundary threads take a branch of their own, and the shifted
    loads straddle 128-byte lines."""
    return HEADER + """\
.visible .entry stencil3(
    .param .u64 param_in,
    .param .u64 param_out,
    .param .u32 param_n
)
{
    .reg .pred %p<3>;
    .reg .b32 %r<12>;
    .reg .b64 %rd<8>;

    ld.param.u64 %rd1, [param_in];
    ld.param.u64 %rd2, [param_out];
    ld.param.u32 %r1, [param_n];
    mov.u32 %r2, %tid.x;
    mov.u32 %r3, %ctaid.x;
    mov.u32 %r4, %ntid.x;
    mad.lo.s32 %r5, %r3, %r4, %r2;
    setp.ge.u32 %p1, %r5, %r1;
    @%p1 bra $L__done;
    mul.wide.u32 %rd3, %r5, 4;
    add.s64 %rd4, %rd1, %rd3;
    add.s64 %rd5, %rd2, %rd3;
    ld.global.u32 %r6, [%rd4];
    add.s32 %r7, %r1, -1;
    setp.eq.u32 %p1, %r5, 0;
    setp.eq.u32 %p2, %r5, %r7;
    @%p1 bra $L__edge;
    @%p2 bra $L__edge;
    ld.global.u32 %r8, [%rd4+-4];
    ld.global.u32 %r9, [%rd4+4];
    add.s32 %r10, %r8, %r6;
    add.s32 %r6, %r10, %r9;
$L__edge:
    st.global.u32 [%rd5], %r6;
$L__done:
    ret;
}
"""


def lcg64_ptx(iters: int = 37) -> str:
    """64-bit integer work per thread: x = seeds[gid] (u64), then `iters` times
    x = x * A + C (mad.lo.u64, A = 6364136223846793005, C = 1442695040888963407);
    then y = x * x + x - C, z = (x < y unsigned) ? x : y, s = (x < y signed) ? 1 : 0;
    out[3 gid .. 3 gid + 2] = x, y, z (u64) and flags[gid] = s (u32).  There is no
    bounds check: the grid must cover the arrays exactly."""
    return HEADER + """\
.visible .entry lcg64(
    .param .u64 param_seeds,
    .param .u64 param_out,
    .param .u64 param_flags
)
{
    .reg .pred %%p<3>;
    .reg .b32 %%r<8>;
    .reg .b64 %%rd<16>;

    ld.param.u64 %%rd1, [param_seeds];
    ld.param.u64 %%rd2, [param_out];
    ld.param.u64 %%rd3, [param_flags];
    mov.u32 %%r1, %%tid.x;
    mov.u32 %%r2, %%ctaid.x;
    mov.u32 %%r3, %%ntid.x;
    mad.lo.s32 %%r4, %%r2, %%r3, %%r1;
    mul.wide.u32 %%rd4, %%r4, 8;
    add.s64 %%rd5, %%rd1, %%rd4;
    ld.global.u64 %%rd6, [%%rd5];
    mov.u64 %%rd7, 6364136223846793005;
    mov.u64 %%rd8, 1442695040888963407;
    mov.u32 %%r5, 0;
$L__loop:
    mad.lo.u64 %%rd6, %%rd6, %%rd7, %%rd8;
    add.s32 %%r5, %%r5, 1;
    setp.lt.s32 %%p1, %%r5, %d;
    @%%p1 bra $L__loop;
    mul.lo.u64 %%rd9, %%rd6, %%rd6;
    add.u64 %%rd9, %%rd9, %%rd6;
    sub.u64 %%rd9, %%rd9, %%rd8;
    setp.lt.u64 %%p1, %%rd6, %%rd9;
    selp.b64 %%rd10, %%rd6, %%rd9, %%p1;
    setp.lt.s64 %%p2, %%rd6, %%rd9;
    selp.b32 %%r6, 1, 0, %%p2;
    mul.wide.u32 %%rd11, %%r4, 24;
    add.s64 %%rd12, %%rd2, %%rd11;
    st.global.u64 [%%rd12], %%rd6;
    st.global.u64 [%%rd12+8], %%rd9;
    st.global.u64 [%%rd12+16], %%rd10;
    mul.wide.u32 %%rd13, %%r4, 4;
    add.s64 %%rd14, %%rd3, %%rd13;
    st.global.u32 [%%rd14], %%r6;
    ret;
}
""" % iters


# (setp form, operands): the comparisons of setp_forms_ptx, result bit k of flags[i]
SETP_FORMS = [("setp.lo.u32", "%r1, %r2"), ("setp.ls.u32", "%r1, %r2"), ("setp.hi.u32", "%r1, %r2"),
              ("setp.hs.u32", "%r1, %r2"), ("setp.eq.b32", "%r1, %r2"), ("setp.ne.b32", "%r1, %r2"),
              ("setp.lo.u64", "%rd7, %rd8"), ("setp.hs.u64", "%rd7, %rd8"), ("setp.eq.b64", "%rd7, %rd8"),
              ("setp.ne.b64", "%rd7, %rd8"), ("setp.le.s32", "%r1, %r2"), ("setp.ge.u32", "%r1, %r2")]


def setp_forms_ptx() -> str:
    """Per thread i: a = A[i], b = B[i] (u32) and c = C[i], d = D[i] (u64); flags[i]
    gets bit k set when comparison k of SETP_FORMS holds; prod[i] = a * b
    (mul.lo.u32) and fma[i] = a * b + a (mad.lo.u32).  Arrays: A, B at 4 i, C, D at
    8 i from their bases; flags at out + 4 i, prod at out + 65536 + 4 i, fma at
    out + 131072 + 4 i."""
    L = [HEADER + ".visible .entry setp_forms(\n    .param .u64 param_a,\n    .param .u64 param_b,\n"
         "    .param .u64 param_c,\n    .param .u64 param_d,\n    .param .u64 param_out\n)\n{",
         "    .reg .pred %p<2>;", "    .reg .b32 %r<12>;", "    .reg .b64 %rd<16>;",
         "    ld.param.u64 %rd1, [param_a];", "    ld.param.u64 %rd2, [param_b];",
         "    ld.param.u64 %rd3, [param_c];", "    ld.param.u64 %rd4, [param_d];",
         "    ld.param.u64 %rd5, [param_out];",
         "    mov.u32 %r3, %tid.x;", "    mov.u32 %r4, %ctaid.x;", "    mov.u32 %r5, %ntid.x;",
         "    mad.lo.u32 %r6, %r4, %r5, %r3;", "    mul.wide.u32 %rd6, %r6, 4;", "    mul.wide.u32 %rd9, %r6, 8;",
         "    add.s64 %rd10, %rd1, %rd6;", "    ld.global.u32 %r1, [%rd10];",
         "    add.s64 %rd10, %rd2, %rd6;", "    ld.global.u32 %r2, [%rd10];",
         "    add.s64 %rd10, %rd3, %rd9;", "    ld.global.u64 %rd7, [%rd10];",
         "    add.s64 %rd10, %rd4, %rd9;", "    ld.global.u64 %rd8, [%rd10];",
         "    mov.u32 %r7, 0;"]
    for k, (form, ops) in enumerate(SETP_FORMS):
        L += ["    %s %%p1, %s;" % (form, ops), "    selp.b32 %%r8, %d, 0, %%p1;" % (1 << k),
              "    add.s32 %r7, %r7, %r8;"]
    L += ["    mul.lo.u32 %r9, %r1, %r2;", "    mad.lo.u32 %r10, %r1, %r2, %r1;",
          "    add.s64 %rd11, %rd5, %rd6;", "    st.global.u32 [%rd11], %r7;",
          "    add.s64 %rd13, %rd5, 65536;", "    add.s64 %rd14, %rd13, %rd6;",
          "    st.global.u32 [%rd14], %r9;", "    add.s64 %rd15, %rd14, 65536;", "    st.global.u32 [%rd15], %r10;",
          "    ret;", "}"]
    return "\n".join(L) + "\n"


def setp_forms_inputs(nt: int, seed: int):
    """Seeded inputs of setp_forms_ptx for nt threads: u32 a, b with every fourth
    pair equal and every eighth (from 1) adjacent, u64 c, d with every third pair
    equal; returns (a, b, c, d, the five parameter offsets, the memory image)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 1 << 32, size=nt, dtype=np.uint32)
    b = rng.integers(0, 1 << 32, size=nt, dtype=np.uint32)
    b[::4] = a[::4]
    b[1::8] = a[1::8] + np.uint32(1)
    c = rng.integers(0, 1 << 64, size=nt, dtype=np.uint64)
    d = rng.integers(0, 1 << 64, size=nt, dtype=np.uint64)
    d[::3] = c[::3]
    offs = (0, 8 * nt, 16 * nt, 32 * nt, 48 * nt)
    g = np.zeros(offs[4] + 3 * 65536, np.uint8)
    for arr, o in zip((a, b, c, d), offs):
        g[o:o + arr.nbytes] = arr.view(np.uint8)
    return a, b, c, d, offs, g


F32_SETP = ["eq", "ne", "lt", "le", "gt", "ge"]


def f32_setp_ptx() -> str:
    """Per thread i: a, b = in[2 i], in[2 i + 1] (f32 bit patterns); flags[i] gets
    bit k set when setp.<F32_SETP[k]>.f32 a, b holds (ordered: false whenever an
    operand is NaN), and pick[i] = selp.f32 of a or b on a < b.  flags at out + 4 i,
    pick at out + 65536 + 4 i; threads at i >= n do nothing."""
    L = [HEADER + ".visible .entry f32_setp(\n    .param .u64 param_in,\n    .param .u64 param_out,\n"
         "    .param .u32 param_n\n)\n{",
         "    .reg .pred %p<3>;", "    .reg .b32 %r<10>;", "    .reg .f32 %f<4>;", "    .reg .b64 %rd<8>;",
         "    ld.param.u64 %rd1, [param_in];", "    ld.param.u64 %rd2, [param_out];", "    ld.param.u32 %r1, [param_n];",
         "    mov.u32 %r2, %tid.x;", "    mov.u32 %r3, %ctaid.x;", "    mov.u32 %r4, %ntid.x;",
         "    mad.lo.s32 %r5, %r3, %r4, %r2;", "    setp.ge.u32 %p2, %r5, %r1;", "    @%p2 bra $L__done;",
         "    mul.wide.u32 %rd3, %r5, 8;", "    add.s64 %rd4, %rd1, %rd3;",
         "    ld.global.f32 %f1, [%rd4];", "    ld.global.f32 %f2, [%rd4+4];", "    mov.u32 %r6, 0;"]
    for k, cmp in enumerate(F32_SETP):
        L += ["    setp.%s.f32 %%p1, %%f1, %%f2;" % cmp, "    selp.b32 %%r7, %d, 0, %%p1;" % (1 << k),
              "    add.s32 %r6, %r6, %r7;"]
    L += ["    setp.lt.f32 %p1, %f1, %f2;", "    selp.f32 %f3, %f1, %f2, %p1;",
          "    mul.wide.u32 %rd5, %r5, 4;", "    add.s64 %rd6, %rd2, %rd5;", "    st.global.u32 [%rd6], %r6;",
          "    add.s64 %rd7, %rd6, 65536;", "    st.global.f32 [%rd7], %f3;", "$L__done:", "    ret;", "}"]
    return "\n".join(L) + "\n"
