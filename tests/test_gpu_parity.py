"""GPU parity: libkscope on gfx950 against the CPU oracle, bit for bit.

Every case runs the same seeded inputs through the C ABI (ks_load_program,
ks_alloc_state, ks_run, ks_read_*) and through the oracle, then compares the
simulated memory, every field of every per-warp counter record, the trace
headers and every written trace record.  The tolerance is zero everywhere: f32
results are IEEE round-to-nearest on both sides (0 ULP), and everything else is
integer.  Full-size workloads are compared on sampled blocks: blocks never
communicate, so the oracle can simulate any subset exactly.
"""
import math
import sys

import numpy as np
import pytest

from workloads import configs as W
from workloads import small as S
from workloads.configs import pack_params

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from analysis_ptxsimulator_amd import ks
    ks.lib()
    return ks


def gpu_run(K, w, trace_cap=None, max_warp_instrs=0xFFFFFFFF, latency=None, runs=1):
    cap = w.trace_cap if trace_cap is None else trace_cap
    _say("%s grid=%s block=%s cap=%d" % (w.name, w.grid, w.block, cap))
    s = K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=cap, max_warp_instrs=max_warp_instrs,
                  latency=latency)
    try:
        outs = []
        for _ in range(runs):
            s.load_gmem(w.gmem)
            s.run(w.params_bytes)
            outs.append((s.read_gmem(), s.read_counters(), s.read_trace(), s.status()))
        return outs if runs > 1 else outs[0]
    finally:
        s.close()


def oracle_run(O, w, trace_cap=None, blocks=None, **kw):
    cap = w.trace_cap if trace_cap is None else trace_cap
    g = w.gmem.copy()
    c, t, _ = O.run(w.ptx, w.grid, w.block, w.params_bytes, g, trace_cap=cap, blocks=blocks, **kw)
    return g, c, t


def compare_counters(cg, co, where=""):
    assert cg.dtype.names == co.dtype.names
    for f in co.dtype.names:
        if not np.array_equal(cg[f], co[f]):
            bad = np.nonzero(cg[f] != co[f])[0][:5]
            raise AssertionError("%s counter %s differs at warps %s: gpu %s oracle %s" %
                                 (where, f, bad.tolist(), cg[f][bad].tolist(), co[f][bad].tolist()))


def compare_traces(K, tg, to, cap, where=""):
    hg, rg = K.trace_slots(tg, cap)
    ho, ro = K.trace_slots(to, cap)
    for f in ho.dtype.names:
        assert np.array_equal(hg[f], ho[f]), "%s trace header %s differs" % (where, f)
    for wi in range(len(ho)):
        n = int(ho["records_written"][wi])
        if not np.array_equal(rg[wi, :n], ro[wi, :n]):
            k = int(np.nonzero((rg[wi, :n] != ro[wi, :n]).any(axis=1))[0][0])
            raise AssertionError("%s warp %d record %d: gpu %s oracle %s" %
                                 (where, wi, k, rg[wi, k].tolist(), ro[wi, k].tolist()))


def full_parity(K, O, w, trace_cap=None, oracle_threads=0, **kw):
    cap = w.trace_cap if trace_cap is None else trace_cap
    gg, cg, tg, st = gpu_run(K, w, trace_cap=cap, **kw)
    okw = {}
    if "max_warp_instrs" in kw:
        okw["max_warp_instrs"] = kw["max_warp_instrs"]
    if "latency" in kw:
        okw["latency"] = kw["latency"]
    if oracle_threads:
        okw["threads"] = oracle_threads
    go, co, to = oracle_run(O, w, trace_cap=cap, **okw)
    if not np.array_equal(gg, go):
        bad = np.nonzero(gg != go)[0]
        raise AssertionError("%s: %d memory bytes differ, first at %d" % (w.name, bad.size, bad[0]))
    compare_counters(cg, co, w.name)
    compare_traces(K, tg, to, cap, w.name)
    assert st == int(np.bitwise_or.reduce(co["status"])) if len(co) else st == 0
    return cg


def sampled_parity(K, O, w, blocks, regions, trace_cap=None):
    """GPU runs the whole grid; the oracle simulates only `blocks`.  Compares the
    sampled blocks' warps and, per region (offset, bytes per thread), the bytes
    those blocks' threads own."""
    cap = w.trace_cap if trace_cap is None else trace_cap
    gg, cg, tg, st = gpu_run(K, w, trace_cap=cap)
    go, co, to = oracle_run(O, w, trace_cap=cap, blocks=blocks)
    wpb = w.warps_per_block
    slot = 16 + 8 * cap
    tg2 = tg.reshape(-1, slot)
    for i, b in enumerate(blocks):
        sl = slice(b * wpb, (b + 1) * wpb)
        compare_counters(cg[sl], co[i * wpb:(i + 1) * wpb], "%s block %d" % (w.name, b))
        compare_traces(K, tg2[sl].reshape(-1), to.reshape(-1, slot)[i * wpb:(i + 1) * wpb].reshape(-1), cap,
                       "%s block %d" % (w.name, b))
        tpb = w.threads_per_block
        for off, per_thread, stride in regions:
            for t0 in (b * tpb,):
                lo = off + t0 * per_thread
                hi = off + (t0 + tpb) * per_thread
                if stride:
                    for j in range(4):
                        lo2, hi2 = lo + j * stride, hi + j * stride
                        assert np.array_equal(gg[lo2:hi2], go[lo2:hi2]), "%s block %d region %d+%d" % (w.name, b, off, j)
                else:
                    assert np.array_equal(gg[lo:hi], go[lo:hi]), "%s block %d region %d" % (w.name, b, off)
    return cg, co


# ------------------------------------------------------------------ small, full comparisons

def test_vector_add(K, oracle_mod):
    cg = full_parity(K, oracle_mod, W.vector_add())
    assert int(cg["thread_instrs"].sum()) == 19264


def test_f32_edge_operands(K, oracle_mod):
    full_parity(K, oracle_mod, S.f32_ops(n=16384))


@pytest.mark.parametrize("s", W.STRIDES)
def test_strided_small(K, oracle_mod, s):
    cg = full_parity(K, oracle_mod, W.strided_gather(s, n=1 << 16))
    assert (cg["gld_sectors"] == min(32, 4 * s) + 4).all()


@pytest.mark.parametrize("n_acc", [1, 2, 3, 8])
def test_ffma_small(K, oracle_mod, n_acc):
    full_parity(K, oracle_mod, W.ffma_probe(n_acc=n_acc, iters=40, grid=6, block=256, trace_cap=600))


@pytest.mark.parametrize("s", list(range(1, 33)))
def test_bank_small(K, oracle_mod, s):
    cg = full_parity(K, oracle_mod, W.bank_probe(s, iters=12, grid=3, block=1024, trace_cap=64))
    assert (cg["sh_degree_max"] == math.gcd(s, 32)).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_stress_small(K, oracle_mod, seed):
    w = W.random_stress(prog_seed=seed, grid=48, block=256, gmem_bytes=1 << 24, trace_cap=2048)
    full_parity(K, oracle_mod, w)


@pytest.mark.parametrize("block", [1024, 992, 96])
def test_random_stress_block_sizes(K, oracle_mod, block):
    """The 64-slot program (72-VGPR register file) on full-size, ragged and small
    blocks: 16 waves per workgroup, a last wave with one warp, one and a half waves."""
    w = W.random_stress(prog_seed=2, grid=12 if block > 256 else 40, block=block, gmem_bytes=1 << 24,
                        trace_cap=512)
    assert K.ks_interp_kernel(K.ks_load_program(w.ptx), w.block) == "ks_interp_v64"
    full_parity(K, oracle_mod, w)


@pytest.mark.parametrize("seed", range(24))
def test_control_flow_shapes(K, oracle_mod, seed):
    rng = np.random.default_rng(seed)
    n = 256
    data = rng.choice([0, 1, 500, 1500, 2500, 2999], size=n).astype(np.uint32)
    g = np.zeros(8 * n + 4096, np.uint8)
    g[:4 * n] = data.view(np.uint8)
    w = W.Workload(name="cfg%d" % seed, ptx=S.random_cfg_ptx(seed), grid=(2, 1, 1), block=(128, 1, 1),
                   params=[("param_in", "u64", 0), ("param_out", "u64", 4 * n)], gmem=g, trace_cap=128)
    full_parity(K, oracle_mod, w)


def test_long_program(K, oracle_mod):
    """A 32000-instruction random program: records read from 4 MB into the decoded
    table, the two-ahead prefetch near its end, and about 31000 issues per warp
    against a 1024-record cap (the rest counted as dropped)."""
    w = W.random_stress(prog_seed=7, grid=2, block=64, gmem_bytes=1 << 22, trace_cap=1024, n_instr=32000)
    cg = full_parity(K, oracle_mod, w, oracle_threads=_host_threads())
    assert (cg["warp_instrs"] > 30000).all()


def test_largest_shared_window(K, oracle_mod):
    """A 65536-byte shared window (the largest a program may declare) used at its
    edges, past its end and misaligned, on 256-thread blocks; where the device's
    LDS cannot hold it beside the scoreboards the run must be refused instead."""
    import struct
    w = W.Workload(name="shared_edges", ptx=S.shared_edges_ptx(), grid=(2, 1, 1), block=(256, 1, 1),
                   params=[("param_out", "u64", 0)], gmem=np.zeros(2 * 256 * 32, np.uint8), trace_cap=64)
    assert w.params_bytes == struct.pack("<Q", 0)
    try:
        cg = full_parity(K, oracle_mod, w)
    except K.KsError as e:  # scoreboards, staging rings and a 64 KiB window beyond the device's LDS
        assert e.code == -2 and "LDS" in e.msg, e
        _say("shared_edges refused: %s" % e.msg)
        return
    assert (cg["fault_n"] == 64).all() and (cg["sh_n"] == 8).all()


@pytest.mark.parametrize("budget", [0, 1])
def test_budget_zero_and_one(K, oracle_mod, budget):
    """An issue budget of 0 stops every warp before its first issue (nothing
    issued, cycles 0, status BUDGET); a budget of 1 lets each warp issue once."""
    cg = full_parity(K, oracle_mod, W.random_stress(prog_seed=3, grid=3, block=96, gmem_bytes=1 << 22, trace_cap=8),
                     max_warp_instrs=budget)
    assert (cg["warp_instrs"] == budget).all() and (cg["status"] & 2).all()


def test_memory_too_small_for_every_access(K, oracle_mod):
    """vector_add over a 4096-byte simulated memory: b and c lie past its end, so
    every access to them faults (loads read 0, stores are dropped) and is still
    analysed, while a stays in range."""
    w = W.vector_add()
    w = W.Workload(name="vector_add_small_mem", ptx=w.ptx, grid=w.grid, block=w.block, params=w.params,
                   gmem=w.gmem[:4096].copy(), trace_cap=w.trace_cap)
    cg = full_parity(K, oracle_mod, w)
    assert (cg["fault_n"] > 0).all() and (cg["status"] & 4).all()


def test_latency_class_of_every_producer(K, oracle_mod):
    """Every destination-writing form of the subset, each followed by a consumer of
    its result, under a latency table of distinct values per class: the GPU's
    issue cycles must equal the oracle's, which its pins fix per class."""
    lat = [101 + 10 * k for k in range(14)] + [28, 150, 400, 0]
    g = np.zeros(4096, np.uint8)
    g[64:72] = np.arange(1, 9, dtype=np.uint8)
    w = W.Workload(name="latency_classes", ptx=S.latency_classes_ptx(), grid=(2, 1, 1), block=(40, 1, 1),
                   params=[("param_p", "u64", 64), ("param_q", "u32", 9)], gmem=g, trace_cap=128)
    full_parity(K, oracle_mod, w, latency=lat)


@pytest.mark.parametrize("block", [64, 256, 1024])
def test_block_reduce(K, oracle_mod, block):
    """A shared-memory tree reduction: barriers between its steps, divergence that
    narrows inside warp 0, stride-1 shared accesses, one output per block."""
    grid = 24
    data = np.random.default_rng(block).integers(0, 1 << 32, size=grid * block, dtype=np.uint32)
    out = 4 * grid * block
    g = np.zeros(out + 4 * grid, np.uint8)
    g[:out] = data.view(np.uint8)
    w = W.Workload(name="block_reduce_%d" % block, ptx=S.block_reduce_ptx(block), grid=(grid, 1, 1),
                   block=(block, 1, 1), params=[("param_in", "u64", 0), ("param_out", "u64", out)], gmem=g,
                   trace_cap=64)
    full_parity(K, oracle_mod, w)


@pytest.mark.parametrize("pad", [0, 1])
def test_tile_transpose(K, oracle_mod, pad):
    """A shared-tile transpose on 32 x 32 blocks over a 4 x 4 grid, with 32-way bank
    conflicts on the unpadded tile's column loads and none on the padded one."""
    gx = 4
    n = 32 * gx
    g = np.zeros(8 * n * n, np.uint8)
    g[:4 * n * n] = np.random.default_rng(pad).integers(0, 1 << 32, size=n * n, dtype=np.uint32).view(np.uint8)
    w = W.Workload(name="tile_transpose_pad%d" % pad, ptx=S.tile_transpose_ptx(pad), grid=(gx, gx, 1),
                   block=(32, 32, 1), params=[("param_in", "u64", 0), ("param_out", "u64", 4 * n * n)], gmem=g,
                   trace_cap=64)
    cg = full_parity(K, oracle_mod, w)
    assert (cg["sh_degree_max"] == (32 if pad == 0 else 1)).all()


def test_stencil3(K, oracle_mod):
    """A 3-point stencil over a ragged n: branches at both ends and past n, loads
    that straddle 128-byte lines."""
    n, block = 100003, 256
    data = np.random.default_rng(17).integers(0, 1 << 32, size=n, dtype=np.uint32)
    off = (4 * n + 4095) // 4096 * 4096
    g = np.zeros(off + 4 * n, np.uint8)
    g[:4 * n] = data.view(np.uint8)
    w = W.Workload(name="stencil3", ptx=S.stencil3_ptx(), grid=((n + block - 1) // block, 1, 1), block=(block, 1, 1),
                   params=[("param_in", "u64", 0), ("param_out", "u64", off), ("param_n", "u32", n)], gmem=g,
                   trace_cap=32)
    full_parity(K, oracle_mod, w)


def test_lcg64(K, oracle_mod):
    """64-bit integer forms in a loop (mad/mul/add/sub.u64, 64-bit setp and selp,
    u64 loads and stores) over 6080 threads (the program has no bounds check, so
    the grid covers the arrays exactly: extra threads would write into the flags
    and race with their owners)."""
    nt, block = 6080, 160
    seeds = np.random.default_rng(21).integers(0, 1 << 64, size=nt, dtype=np.uint64)
    so, oo, fo = 0, 8 * nt, 32 * nt
    g = np.zeros(fo + 4 * nt, np.uint8)
    g[:8 * nt] = seeds.view(np.uint8)
    w = W.Workload(name="lcg64", ptx=S.lcg64_ptx(), grid=((nt + block - 1) // block, 1, 1), block=(block, 1, 1),
                   params=[("param_seeds", "u64", so), ("param_out", "u64", oo), ("param_flags", "u64", fo)],
                   gmem=g, trace_cap=64)
    full_parity(K, oracle_mod, w)


def test_setp_forms(K, oracle_mod):
    """The unsigned setp mnemonics, eq/ne on .bN, 64-bit compares and the .u32
    multiply forms over 8192 threads with equal and adjacent input pairs."""
    nt = 8192
    a, b, c, d, offs, g = S.setp_forms_inputs(nt, 31)
    w = W.Workload(name="setp_forms", ptx=S.setp_forms_ptx(), grid=(nt // 256, 1, 1), block=(256, 1, 1),
                   params=[(n, "u64", o) for n, o in zip(("param_a", "param_b", "param_c", "param_d", "param_out"),
                                                           offs)], gmem=g, trace_cap=32)
    full_parity(K, oracle_mod, w)


def test_f32_setp(K, oracle_mod):
    """setp.*.f32 and selp.f32 over the f32 edge values and random patterns."""
    ops = S.f32_operands(16384, 13)[:, :2].copy()
    n = len(ops)
    out = 8 * n + 4096
    g = np.zeros(out + 65536 + 4 * n, np.uint8)
    g[:8 * n] = ops.reshape(-1).view(np.uint8)
    w = W.Workload(name="f32_setp", ptx=S.f32_setp_ptx(), grid=((n + 255) // 256, 1, 1), block=(256, 1, 1),
                   params=[("param_in", "u64", 0), ("param_out", "u64", out), ("param_n", "u32", n)], gmem=g,
                   trace_cap=16)
    full_parity(K, oracle_mod, w)


def test_single_ret_program(K, oracle_mod):
    """The smallest program (a lone ret, no parameters) on 33-thread blocks: a full
    warp and a one-lane warp per block."""
    w = W.Workload(name="ret_only", ptx=S.HEADER + ".visible .entry k()\n{\n    ret;\n}\n", grid=(3, 1, 1),
                   block=(33, 1, 1), params=[], gmem=np.zeros(64, np.uint8), trace_cap=4)
    cg = full_parity(K, oracle_mod, w)
    assert list(cg["thread_instrs"]) == [32, 1] * 3 and (cg["cycles"] == 1).all()


def test_staircase_depth_63(K, oracle_mod):
    g = np.zeros(4096, np.uint8)
    w = W.Workload(name="staircase", ptx=S.staircase_ptx(31), grid=(2, 1, 1), block=(96, 1, 1),
                   params=[("param_out", "u64", 0)], gmem=g, trace_cap=256)
    cg = full_parity(K, oracle_mod, w)
    assert cg["max_stack_depth"].max() == 63


def test_analyser_vectors(K, oracle_mod):
    rng = np.random.default_rng(17)
    n = 256 * 8
    base = rng.integers(0, 1 << 12, size=n // 32) * 4
    kinds = np.arange(n // 32) % 6
    ga, sa = [], []
    for k, b0 in zip(kinds, base):
        lanes = np.arange(32)
        if k == 0:
            g = b0 + 4 * lanes * int(rng.integers(0, 40))
        elif k == 1:
            g = rng.integers(0, 1 << 14, size=32) * 4
        elif k == 2:
            g = np.full(32, b0)
        elif k == 3:
            g = b0 + 4 * rng.permutation(32)
        elif k == 4:
            g = b0 + 2 * lanes  # misaligned lanes: faults, both end sectors counted
        else:
            g = np.where(rng.random(32) < 0.2, (1 << 17) + 64 * lanes, b0 + 4 * lanes)  # some out of range
        ga.append(g)
        sa.append((4 * int(rng.integers(0, 33)) * lanes + int(rng.integers(0, 4)) * 4) % 4096)
    guard = (rng.random(n) < 0.8).astype(np.uint32)
    w = S.addr_probe(np.concatenate(ga).astype(np.uint64), np.concatenate(sa).astype(np.uint32), guard, 1 << 16)
    full_parity(K, oracle_mod, w)


# ------------------------------------------------------------------ edge cases

def test_ragged_and_3d_shapes(K, oracle_mod):
    ptx = S.random_cfg_ptx(3)
    for grid, block in [((3, 2, 1), (100, 1, 1)), ((1, 1, 1), (33, 1, 1)), ((2, 1, 2), (8, 4, 3)),
                        ((1, 1, 1), (1024, 1, 1)), ((5, 1, 1), (1, 1, 1))]:
        nt = grid[0] * grid[1] * grid[2] * block[0] * block[1] * block[2]
        rng = np.random.default_rng(nt)
        g = np.zeros(8 * nt + 4096, np.uint8)
        g[:4 * nt] = rng.choice([0, 1, 500, 1500, 2500], size=nt).astype(np.uint32).view(np.uint8)
        w = W.Workload(name="shape%s%s" % (grid, block), ptx=ptx, grid=grid, block=block,
                       params=[("param_in", "u64", 0), ("param_out", "u64", 4 * nt)], gmem=g, trace_cap=64)
        full_parity(K, oracle_mod, w)


def test_budget_trace_cap_and_latency_table(K, oracle_mod):
    w = W.ffma_probe(n_acc=4, iters=12, grid=2, block=256, trace_cap=100)
    full_parity(K, oracle_mod, w, max_warp_instrs=150)
    full_parity(K, oracle_mod, w, trace_cap=0)
    lat = oracle_mod.default_latency()
    lat[2] = 7  # fp32
    lat[7] = 333
    full_parity(K, oracle_mod, w, latency=lat)


def test_cycle_overflow(K, oracle_mod):
    ptx = S.HEADER + """.visible .entry o(.param .u64 param_out)
{
    .reg .pred %p<2>;
    .reg .b32 %r<4>;
    .reg .b64 %rd<2>;
    ld.param.u64 %rd1, [param_out];
    mov.u32 %r2, 0;
$L__loop:
    ld.global.u32 %r1, [%rd1];
    add.s32 %r2, %r2, %r1;
    setp.lt.u32 %p1, %r2, 1;
    @%p1 bra $L__loop;
    ret;
}
"""
    w = W.Workload(name="overflow", ptx=ptx, grid=(1, 1, 1), block=(64, 1, 1), params=[("param_out", "u64", 0)],
                   gmem=np.zeros(64, np.uint8), trace_cap=8)
    lat = oracle_mod.default_latency()
    lat[7] = 65535
    cg = full_parity(K, oracle_mod, w, latency=lat)
    assert (cg["status"] & K.ST_CYCLE_OVF).all()


def test_barrier_in_divergent_region(K, oracle_mod):
    ptx = S.HEADER + """.visible .entry b(.param .u64 param_out)
{
    .reg .pred %p<2>;
    .reg .b32 %r<3>;
    mov.u32 %r1, %laneid;
    setp.lt.u32 %p1, %r1, 8;
    @%p1 bra $L__skip;
    bar.sync 0;
$L__skip:
    ret;
}
"""
    w = W.Workload(name="bardiv", ptx=ptx, grid=(1, 1, 1), block=(200, 1, 1), params=[("param_out", "u64", 0)],
                   gmem=np.zeros(64, np.uint8), trace_cap=8)
    cg = full_parity(K, oracle_mod, w)
    # warps 0-5 reach bar.sync with lanes 0-7 gone; warp 6 (threads 192-199) skips it entirely
    assert (cg["status"][:6] & K.ST_BARDIV).all() and not (cg["status"][6] & K.ST_BARDIV)


def test_last_issue_a_barrier(K, oracle_mod):
    """cycles = last issue + 1 also when a warp's last issue is a bar.sync whose
    release comes later: here the fast warp of each block reaches the barrier at
    cycle 9 and the program ends there, while the slow warp waits for a global
    load first (the release, at 234, raises no issue of the fast warp)."""
    ptx = S.HEADER + """.visible .entry bar_end(.param .u64 param_in)
{
    .reg .pred %p<2>;
    .reg .b32 %r<4>;
    .reg .b64 %rd<3>;
    mov.u32 %r0, %tid.x;
    setp.lt.u32 %p0, %r0, 32;
    @!%p0 bra JOIN;
    ld.param.u64 %rd0, [param_in];
    ld.global.u32 %r1, [%rd0];
    add.s32 %r2, %r1, 1;
JOIN:
    bar.sync 0;
}
"""
    w = W.Workload(name="bar_end", ptx=ptx, grid=(2, 1, 1), block=(64, 1, 1), params=[("param_in", "u64", 0)],
                   gmem=np.zeros(64, np.uint8), trace_cap=16)
    cg = full_parity(K, oracle_mod, w)
    assert cg["cycles"].tolist() == [215, 10, 215, 10]


def test_budget_stop_at_a_barrier(K, oracle_mod):
    """Warps that reach their issue budget exactly at a bar.sync: the release that
    follows is not part of their cycles (a randomised case that found the
    difference: some warps' 777th issue is a barrier)."""
    w = W.random_stress(prog_seed=989, grid=30, block=64, gmem_bytes=1 << 22, trace_cap=33, n_instr=1106)
    cg = full_parity(K, oracle_mod, w, max_warp_instrs=777)
    assert ((cg["status"] & K.ST_BUDGET) != 0).sum() > 0


def test_runs_are_deterministic_and_rerunnable(K, oracle_mod):
    w = W.random_stress(prog_seed=1, grid=16, block=256, gmem_bytes=1 << 24, trace_cap=256)
    outs = gpu_run(K, w, runs=2)
    for a, b in zip(outs[0], outs[1]):
        if isinstance(a, np.ndarray):
            assert np.array_equal(a, b)
        else:
            assert a == b


# ------------------------------------------------------------------ full-size workloads, sampled

def test_vector_add_full_config(K, oracle_mod):
    full_parity(K, oracle_mod, W.vector_add())


@pytest.mark.parametrize("s", W.STRIDES)
def test_strided_full_size(K, oracle_mod, s):
    w = W.strided_gather(s)
    blocks = [0, 1, 2047, 4095] + [int(x) for x in np.random.default_rng(s).integers(0, 4096, 4)]
    n = w.meta["n"]
    off_c = w.outputs["c"][0]
    sampled_parity(K, oracle_mod, w, blocks, [(off_c, 4, 0)])


@pytest.mark.parametrize("n_acc", [1, 8])
def test_ffma_full_size(K, oracle_mod, n_acc):
    w = W.ffma_probe(n_acc=n_acc)
    cg, co = sampled_parity(K, oracle_mod, w, [0, 1023], [(w.outputs["out"][0], 4, 0)])
    # 4096 iterations: 128 (dependent) or 35 (independent) cycles each, plus a fixed prologue/epilogue
    per_iter = 128 if n_acc == 1 else 35
    assert (cg["cycles"] > per_iter * 4096).all() and (cg["cycles"] < per_iter * 4096 + 2000).all()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("s", list(range(1, 33)))
def test_bank_full_size(K, oracle_mod, s):
    """The full 256 x 1024 bank probe at every word stride: all memory, every
    counter record and every trace record against the oracle's full grid."""
    w = W.bank_probe(s)
    cg = full_parity(K, oracle_mod, w, oracle_threads=_host_threads())
    assert (cg["sh_degree_max"] == math.gcd(s, 32)).all()
    assert (cg["sh_degree_sum"] == 2048 * math.gcd(s, 32)).all()


def _host_threads():
    import os
    return max(1, min(16, os.cpu_count() or 1))


def compare_records_masked(rg, ro, n, where):
    """Basic records [warps, cap, 2] of both sides over each warp's first n[w]."""
    cap = ro.shape[1]
    live = np.arange(cap)[None, :] < n.astype(np.int64)[:, None]
    if np.array_equal(np.where(live[:, :, None], rg, 0), np.where(live[:, :, None], ro, 0)):
        return
    diff = (rg != ro).any(axis=2) & live
    wi, k = (int(x[0]) for x in np.nonzero(diff))
    raise AssertionError("%s warp %d record %d: gpu %s oracle %s" % (where, wi, k, rg[wi, k].tolist(),
                                                                     ro[wi, k].tolist()))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_stress_full_size(K, oracle_mod, seed):
    """The timed configuration, 65536 x 256 threads over 1 GiB, on the whole grid:
    the oracle simulates every block (in chunks of 8192 blocks, its memory image
    carried from chunk to chunk: blocks never communicate), and every byte of
    simulated memory (the W1 and W4 output regions included), all 524288 counter
    records, every trace header and every written trace record must agree."""
    w = W.random_stress(prog_seed=seed)
    cap = w.trace_cap
    slot = 16 + 8 * cap
    wpb = w.warps_per_block
    s = K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=cap)
    try:
        _say("random_stress seed %d: full grid %s x %s on the GPU" % (seed, w.grid, w.block))
        s.load_gmem(w.gmem)
        # the kernel never writes a slot past its records_written records: with the
        # buffer cleared first, each slot must equal the oracle's (zero-filled) byte
        # for byte
        s.trace.zero_()
        s.run(w.params_bytes)
        gg = s.read_gmem()
        cg = s.read_counters()
        st = s.status()
        go = w.gmem.copy()
        chunk = 8192
        threads = _host_threads()
        for b0 in range(0, w.n_blocks, chunk):
            blocks = list(range(b0, min(w.n_blocks, b0 + chunk)))
            co, to, _ = oracle_mod.run(w.ptx, w.grid, w.block, w.params_bytes, go, trace_cap=cap, blocks=blocks,
                                       threads=threads)
            wlo, nw = b0 * wpb, len(blocks) * wpb
            where = "random_stress seed %d blocks %d-%d" % (seed, blocks[0], blocks[-1])
            compare_counters(cg[wlo:wlo + nw], co, where)
            tg = s.read_trace(wlo, nw)
            if not np.array_equal(tg, to):
                hg, rg = K.trace_slots(tg, cap)
                ho, ro = K.trace_slots(to, cap)
                for f in ho.dtype.names:
                    assert np.array_equal(hg[f], ho[f]), "%s trace header %s differs" % (where, f)
                compare_records_masked(rg, ro, ho["records_written"], where)
                raise AssertionError("%s: bytes past records_written were written" % where)
            del tg, to
            _say("%s: counters, headers and records equal" % where)
        if not np.array_equal(gg, go):
            bad = np.nonzero(gg != go)[0]
            raise AssertionError("random_stress seed %d: %d memory bytes differ, first at %d" % (seed, bad.size, bad[0]))
        assert st == int(np.bitwise_or.reduce(cg["status"]))
        _say("random_stress seed %d: all 1 GiB of memory equal, status %#x" % (seed, st))
    finally:
        s.close()
