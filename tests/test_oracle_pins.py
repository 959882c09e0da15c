"""Pins of the CPU oracle against facts fixed outside it.

Each test ties one part of the oracle to something it cannot agree with by
construction: exact IEEE-754 rounding computed from rationals, closed forms of
the pages' probes, brute force over small cases, a scalar per-thread reference,
and the worked examples printed on the pages (fixtures under tests/golden/).
"""
import json
import math
import os

import numpy as np
import pytest

from workloads import configs as W
from workloads import small as S
from workloads.configs import pack_params

from . import ieee32
from . import scalar_ref

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run(O, w, **kw):
    g = w.gmem.copy()
    c, t, rc = O.run(w.ptx, w.grid, w.block, w.params_bytes, g, trace_cap=kw.pop("trace_cap", w.trace_cap), **kw)
    return g, c, t, rc


# ------------------------------------------------------------------ P1 arithmetic

def test_f32_arithmetic_exact_rounding(oracle_mod):
    """add/sub/mul/fma.rn.f32 equal the exact rational result rounded to binary32
    (RNE), with subnormals kept and NaN results canonical, on edge crossings and
    random patterns."""
    w = S.f32_ops(n=4096)
    g, c, _, _ = run(oracle_mod, w)
    ins = w.output(g, "in").reshape(-1, 3)
    out = w.output(g, "out").reshape(-1, 4)
    bad = []
    for i in range(len(ins)):
        a, b, cc = (int(x) for x in ins[i])
        exp = (ieee32.add(a, b), ieee32.sub(a, b), ieee32.mul(a, b), ieee32.fma(a, b, cc))
        got = tuple(int(x) for x in out[i])
        if exp != got:
            bad.append((hex(a), hex(b), hex(cc), [hex(x) for x in exp], [hex(x) for x in got]))
    assert not bad, bad[:5]


def test_f32_add_mul_match_numpy_float32(oracle_mod):
    """Textbook special case: numpy float32 add/mul (IEEE, round to nearest) agree
    bit for bit with the oracle on 65536 random operand pairs (NaNs canonicalised)."""
    rng = np.random.default_rng(99)
    n = 65536
    ops = rng.integers(0, 1 << 32, size=(n, 3), dtype=np.uint32)
    w = S.f32_ops(n=8)
    size = W._align(12 * n) + 16 * n
    g = np.zeros(size, dtype=np.uint8)
    g[:12 * n] = ops.reshape(-1).view(np.uint8)
    params = pack_params([("param_in", "u64", 0), ("param_out", "u64", W._align(12 * n)), ("param_n", "u32", n)])
    oracle_mod.run(w.ptx, n // 256, 256, params, g)
    out = g[W._align(12 * n):].view("<u4").reshape(-1, 4)
    a = ops[:, 0].view(np.float32)
    b = ops[:, 1].view(np.float32)
    with np.errstate(all="ignore"):
        for k, ref in ((0, a + b), (1, a - b), (2, a * b)):
            rb = ref.view(np.uint32).copy()
            rb[np.isnan(ref)] = 0x7FFFFFFF
            assert np.array_equal(out[:, k], rb)


# ------------------------------------------------------------------ P2, P3 vector_add

def test_vector_add_values_and_counters(oracle_mod):
    w = W.vector_add()
    g, c, _, _ = run(oracle_mod, w)
    a, b, cc = w.output(g, "a"), w.output(g, "b"), w.output(g, "c")
    assert np.array_equal(cc.view(np.uint32), (a + b).view(np.uint32))
    assert len(c) == 32
    full, tail = c[:31], c[31]
    assert (full["thread_instrs"] == 608).all() and tail["thread_instrs"] == 416
    assert c["thread_instrs"].sum() == 19264
    # a, b, c are 4 KiB aligned: each full-warp access is 4 sectors in 1 line
    assert (full["gld_n"] == 2).all() and (full["gld_sectors"] == 8).all() and (full["gld_lines"] == 2).all()
    assert (full["gst_n"] == 1).all() and (full["gst_sectors"] == 4).all() and (full["gst_lines"] == 1).all()
    assert (full["diverge_n"] == 0).all()
    # warp 31: lanes 0..7 live -> 1 sector, 1 line per access, one divergence
    assert tail["gld_sectors"] == 2 and tail["gld_lines"] == 2 and tail["gst_sectors"] == 1
    assert tail["diverge_n"] == 1
    assert (c["status"] == oracle_mod.ST_FINISHED).all()


def test_vector_add_trace_hand_derived(oracle_mod):
    """Issue cycles derived by hand from the listing and the default latency table
    (tests/golden/vector_add_trace.json)."""
    with open(os.path.join(GOLDEN, "vector_add_trace.json")) as f:
        gold = json.load(f)
    w = W.vector_add()
    _, c, t, _ = run(oracle_mod, w)
    hdr, rec = oracle_mod.trace_slots(t, w.trace_cap)
    for wi in range(32):
        assert hdr[wi]["records_written"] == 19 and hdr[wi]["records_dropped"] == 0
        assert rec[wi, :19, 0].tolist() == gold["issue_cycles"]
        assert rec[wi, :19, 1].tolist() == list(range(19))
        assert hdr[wi]["version"] == 1 and hdr[wi]["warp_in_block"] == wi % 8
        assert hdr[wi]["flags"] == 8
    assert (c["cycles"] == gold["cycles"]).all()


# ------------------------------------------------------------------ P4 - P6 cycle model

@pytest.mark.parametrize("n", [1, 2, 7, 64])
def test_dependent_chain_costs_n_times_latency(oracle_mod, n):
    ptx = S.fma_chain_ptx(n, 1)
    g = np.zeros(64, np.uint8)
    _, t, _ = oracle_mod.run(ptx, 1, 32, pack_params([("param_out", "u64", 0)]), g, trace_cap=n + 8)
    _, rec = oracle_mod.trace_slots(t, n + 8)
    first_fma = rec[0, 3, 0]
    st = rec[0, 3 + n, 0]
    assert st - first_fma == 4 * n


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 8, 16])
def test_accumulator_sweep_cpi(oracle_mod, k):
    """FMA i of a chain over k accumulators issues at 4 * (i // k) + i % k when
    k <= 4 and at i otherwise: in-chain CPI = max(1, 4 / k)."""
    n = 48
    ptx = S.fma_chain_ptx(n, k)
    g = np.zeros(64, np.uint8)
    _, t, _ = oracle_mod.run(ptx, 1, 32, pack_params([("param_out", "u64", 0)]), g, trace_cap=n + 8)
    _, rec = oracle_mod.trace_slots(t, n + 8)
    issues = rec[0, 3:3 + n, 0].astype(int) - int(rec[0, 3, 0])
    exp = [4 * (i // k) + i % k if k <= 4 else i for i in range(n)]
    assert issues.tolist() == exp


@pytest.mark.parametrize("n_acc,slope", [(1, 128), (8, 35)])
def test_count_sweep_exactly_affine(oracle_mod, n_acc, slope):
    """Simulated cycles of the FMA probe loop are exactly affine in the iteration
    count (the simulator's version of the page's T(N) = L N + C regression)."""
    xs = [1, 2, 3, 5, 8, 13]
    ys = []
    for it in xs:
        w = W.ffma_probe(n_acc=n_acc, iters=it, grid=1, block=32, trace_cap=4)
        _, c, _, _ = run(oracle_mod, w)
        ys.append(int(c["cycles"][0]))
    diffs = [(ys[i + 1] - ys[i]) / (xs[i + 1] - xs[i]) for i in range(len(xs) - 1)]
    assert all(d == slope for d in diffs), (ys, diffs)
    # P2's measured contrast: ~4 cycles per dependent FFMA, ~1 per independent one
    assert slope / 32 == (4.0 if n_acc == 1 else 35 / 32)


def test_cycles_end_at_the_last_issue_not_at_a_later_release(oracle_mod):
    """cycles = last issue + 1 (the cycle model's definition), also for a warp
    whose last issue is a bar.sync released later.  Worked by hand with the
    default latencies (mov, setp and add 4, ld.param 4, ld.global 200, bar.sync
    20): the warp of threads 0-31 issues mov 0, setp 4, bra 8, ld.param 9,
    ld.global 13, add 213, bar.sync 214 (cycles 215); the warp of threads 32-63
    branches straight to the barrier: mov 0, setp 4, bra 8, bar.sync 9 (cycles
    10).  The release at 214 + 20 = 234 comes after both warps' last issue: the
    program ends at the barrier."""
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
    g = np.zeros(64, np.uint8)
    c, t, _ = oracle_mod.run(ptx, (2, 1, 1), (64, 1, 1), np.zeros(8, np.uint8).tobytes(), g, trace_cap=16)
    h, r = oracle_mod.trace_slots(t, 16)
    assert c["cycles"].tolist() == [215, 10, 215, 10]
    assert c["warp_instrs"].tolist() == [7, 4, 7, 4]
    assert [int(x) for x in r[0, :7, 0]] == [0, 4, 8, 9, 13, 213, 214]
    assert [int(x) for x in r[1, :4, 0]] == [0, 4, 8, 9] and [int(x) for x in r[1, :4, 1]] == [0, 1, 2, 6]


def test_barrier_release_hand_derived(oracle_mod):
    """bar.sync release = latest arrival of the waiting warps + lat(bar.sync), and a
    warp that finished without reaching the barrier does not hold it: issue cycles
    derived by hand (tests/golden/barrier_trace.json)."""
    with open(os.path.join(GOLDEN, "barrier_trace.json")) as f:
        gold = json.load(f)
    g = np.zeros(64, np.uint8)
    c, t, _ = oracle_mod.run(gold["ptx"], 1, gold["block"], pack_params([("param_out", "u64", 0)]), g,
                             trace_cap=16)
    hdr, rec = oracle_mod.trace_slots(t, 16)
    for w in range(3):
        pcs, cyc = gold["pcs"][str(w)], gold["issue_cycles"][str(w)]
        n = len(pcs)
        assert hdr[w]["records_written"] == n
        assert rec[w, :n, 1].tolist() == pcs, (w, rec[w, :n].tolist())
        assert rec[w, :n, 0].tolist() == cyc, (w, rec[w, :n].tolist())
        assert c["cycles"][w] == gold["cycles"][str(w)]
        assert c["barrier_n"][w] == gold["barrier_n"][str(w)]
        assert c["warp_instrs"][w] == n and c["stall_cycles"][w] == c["cycles"][w] - n
    assert (c["status"] == oracle_mod.ST_FINISHED).all() and (c["diverge_n"] == 0).all()


def _barrier_chain_ptx(k, slow_warp):
    body = []
    for j in range(k):
        body += ["    @%%p1 bra $L__b%d;" % j, "    ld.global.u32 %r2, [%rd1];", "    add.s32 %r3, %r3, %r2;",
                 "$L__b%d:" % j, "    bar.sync 0;"]
    cmp = "ge" if slow_warp == 0 else "lt"
    return S.HEADER + """.visible .entry barchain(.param .u64 param_out)
{
    .reg .pred %%p<2>;
    .reg .b32 %%r<4>;
    .reg .b64 %%rd<2>;
    ld.param.u64 %%rd1, [param_out];
    mov.u32 %%r1, %%tid.x;
    setp.%s.u32 %%p1, %%r1, 32;
%s
    ret;
}
""" % (cmp, "\n".join(body))


@pytest.mark.parametrize("slow_warp", [0, 1])
@pytest.mark.parametrize("k", [1, 2, 3, 7, 20])
def test_barrier_chain_closed_form(oracle_mod, k, slow_warp):
    """k barriers, one warp running a 200-cycle load before each: both warps finish
    at cycles = 10 + 222 k (hand-derived in tests/golden/barrier_trace.json,
    'chain'), whichever warp is the slow one."""
    with open(os.path.join(GOLDEN, "barrier_trace.json")) as f:
        gold = json.load(f)["chain"]
    g = np.zeros(64, np.uint8)
    c, t, _ = oracle_mod.run(_barrier_chain_ptx(k, slow_warp), 1, gold["block"],
                             pack_params([("param_out", "u64", 0)]), g, trace_cap=8 * k + 8)
    assert c["cycles"].tolist() == [gold["cycles_at_zero"] + gold["cycles_per_barrier"] * k] * 2
    assert c["barrier_n"].tolist() == [k, k]
    fast = 1 - slow_warp
    assert c["warp_instrs"][slow_warp] == 4 * k + 4 and c["warp_instrs"][fast] == 2 * k + 4
    # iteration j's bra (pc 3 + 4 j) issues at t_j = 9 + 222 j in both warps, and
    # the final ret at 9 + 222 k
    _, rec = oracle_mod.trace_slots(t, 8 * k + 8)
    for w in range(2):
        n = int(c["warp_instrs"][w])
        at = {int(p): int(cy) for cy, p in rec[w, :n].tolist()}
        assert [at[3 + 4 * j] for j in range(k)] == [9 + 222 * j for j in range(k)]
        assert rec[w, n - 1].tolist() == [9 + 222 * k, 3 + 4 * k]


def test_ffma_probe_values(oracle_mod):
    """Probe outputs equal the scalar reference (exact IEEE fma) for a few threads."""
    for n_acc in (1, 8):
        w = W.ffma_probe(n_acc=n_acc, iters=3, grid=1, block=32, trace_cap=4)
        g, _, _, _ = run(oracle_mod, w)
        g2 = w.gmem.copy()
        scalar_ref.run_grid(w.ptx, w.grid, w.block, w.params_bytes, g2)
        assert np.array_equal(g, g2)


# ------------------------------------------------------------------ P7 strided sectors

@pytest.mark.parametrize("s", W.STRIDES)
def test_strided_sectors_lines_closed_form(oracle_mod, s):
    w = W.strided_gather(s, n=2048)
    g, c, _, _ = run(oracle_mod, w)
    assert (c["gld_n"] == 2).all()
    assert (c["gld_sectors"] == min(32, 4 * s) + 4).all()
    assert (c["gld_lines"] == min(32, s) + 1).all()
    assert (c["gst_n"] == 1).all() and (c["gst_sectors"] == 4).all() and (c["gst_lines"] == 1).all()
    a, b, cc = w.output(g, "a"), w.output(g, "b"), w.output(g, "c")
    assert np.array_equal(cc.view(np.uint32), (a[::s][:2048] + b).view(np.uint32))


# ------------------------------------------------------------------ P8, P9 bank probe

@pytest.mark.parametrize("s", list(range(1, 33)))
def test_bank_degree_is_gcd(oracle_mod, s):
    iters = 3
    w = W.bank_probe(s, iters=iters, grid=2, block=1024, trace_cap=8)
    g, c, _, _ = run(oracle_mod, w)
    d = math.gcd(s, 32)
    assert (c["sh_n"] == 2 * iters).all()
    assert (c["sh_degree_max"] == d).all()
    assert (c["sh_degree_sum"] == 2 * iters * d).all()
    assert (c["barrier_n"] == iters).all()
    v = w.output(g, "v").view(np.uint32).astype(np.uint64)
    out = w.output(g, "out")
    lane = np.arange(2048) % 32
    assert np.array_equal(out, ((iters * v[lane * s]) % (1 << 32)).astype(np.uint32))


# ------------------------------------------------------------------ page examples, P10 brute force

def _bank_degree_page_rule(addrs):
    # restated from the KernelScope memory-analysis description: group active
    # lanes by bank; a bank whose lanes all use one address is a broadcast;
    # degree = largest lane count of a non-broadcast bank, at least 1.
    banks = {}
    for a in addrs:
        banks.setdefault((a // 4) % 32, []).append(a)
    deg = 1
    for lst in banks.values():
        if len(lst) > 1 and len(set(lst)) > 1:
            deg = max(deg, len(lst))
    return deg


def _analyse_with_oracle(O, gaddr, saddr, guard, data_bytes=1 << 16):
    """Counters of the probed accesses alone: the probe program's own table loads
    and output store are removed by subtracting a run with every guard off."""
    blk = 32 * max(1, min(8, len(gaddr) // 32))
    mk = lambda gd: S.addr_probe(np.asarray(gaddr, np.uint64), np.asarray(saddr, np.uint32),
                                 np.asarray(gd, np.uint32), data_bytes, block=blk)
    _, c, _, _ = run(O, mk(guard))
    _, c0, _, _ = run(O, mk(np.zeros(len(guard), np.uint32)))
    out = c.copy()
    for f in ("gld_n", "gld_sectors", "gld_lines", "gst_n", "gst_sectors", "gst_lines", "sh_n",
              "sh_degree_sum"):
        out[f] = c[f] - c0[f]
    return out


def test_page_examples_memory(oracle_mod):
    """Worked examples of the KernelScope memory-analysis part
    (tests/golden/memory_examples.json)."""
    with open(os.path.join(GOLDEN, "memory_examples.json")) as f:
        gold = json.load(f)
    for ex in gold["examples"]:
        addrs = ex["addresses"]
        lanes = len(addrs)
        gaddr = list(addrs) + [0] * (32 - lanes)
        guard = [1] * lanes + [0] * (32 - lanes)
        saddr = [a % 4096 for a in gaddr]
        c = _analyse_with_oracle(oracle_mod, gaddr, saddr, guard)[0]
        if "lines" in ex:
            assert c["gld_lines"] == ex["lines"], ex
            assert c["gld_sectors"] == ex["sectors"], ex
        if "bank_degree" in ex:
            assert c["sh_degree_max"] == ex["bank_degree"], ex


def test_analyser_brute_force(oracle_mod):
    """Random and structured address vectors and masks: sectors/lines equal
    len(set(...)) and the bank degree equals the page rule restated above."""
    rng = np.random.default_rng(5)
    vecs = []
    for k in range(256):
        kind = k % 8
        base = int(rng.integers(0, 1 << 14)) * 4
        if kind == 0:
            g = base + 4 * np.arange(32) * int(rng.integers(0, 40))
        elif kind == 1:
            g = rng.integers(0, 1 << 14, size=32) * 4
        elif kind == 2:
            g = np.full(32, base)
        elif kind == 3:
            g = base + 4 * rng.permutation(32)
        elif kind == 4:
            g = base + 4 * (np.arange(32) // int(rng.integers(1, 9)))
        elif kind == 5:
            g = base + 4 * rng.integers(0, 64, size=32)
        elif kind == 6:
            g = np.sort(rng.integers(0, 1 << 12, size=32)) * 4
        else:
            g = base + 32 * np.arange(32) + 4 * rng.integers(0, 8, size=32)
        s = rng.integers(0, 1024, size=32) * 4 if kind in (1, 5) else (4 * int(rng.integers(0, 33)) * np.arange(32)) % 4096
        if kind == 2:
            s = np.full(32, int(rng.integers(0, 1024)) * 4)
        m = rng.random(32) < (1.0 if k % 3 == 0 else rng.random())
        vecs.append((g % (1 << 16), s, m.astype(np.uint32)))
    gaddr = np.concatenate([v[0] for v in vecs])
    saddr = np.concatenate([v[1] for v in vecs])
    guard = np.concatenate([v[2] for v in vecs])
    c = _analyse_with_oracle(oracle_mod, gaddr, saddr, guard)
    for i, (g, s, m) in enumerate(vecs):
        act = [int(x) for x, on in zip(g, m) if on]
        sact = [int(x) for x, on in zip(s, m) if on]
        if not act:
            assert c[i]["gld_n"] == 0 and c[i]["sh_n"] == 0
            continue
        assert c[i]["gld_n"] == 1 and c[i]["gst_n"] == 1 and c[i]["sh_n"] == 2
        assert c[i]["gld_sectors"] == len({a // 32 for a in act})
        assert c[i]["gld_lines"] == len({a // 128 for a in act})
        assert c[i]["gst_sectors"] == c[i]["gld_sectors"]
        d = _bank_degree_page_rule(sact)
        assert c[i]["sh_degree_max"] == d and c[i]["sh_degree_sum"] == 2 * d


def test_analyser_counts_faulting_and_misaligned_lanes(oracle_mod):
    """Out-of-range and misaligned accesses are analysed (both end sectors of a
    misaligned access count), load 0, store nothing and count as faults."""
    data = 1 << 16
    gaddr = np.array([0, 2, 30, data + 64] + [0] * 28, np.uint64)
    guard = np.array([1, 1, 1, 1] + [0] * 28, np.uint32)
    saddr = np.zeros(32, np.uint32)
    c = _analyse_with_oracle(oracle_mod, gaddr, saddr, guard, data_bytes=data)[0]
    # lane 0: bytes [0,3] sector 0; lane 1: [2,5] misaligned, sector 0; lane 2: [30,33]
    # misaligned, sectors 0 and 1; lane 3: a valid word past the data region
    assert c["gld_sectors"] == len({0, 1, (data + 64) // 32})
    assert c["gld_lines"] == len({0, (data + 64) // 128})
    assert c["fault_n"] == 2 * 2  # lanes 1 and 2, on the load and on the store
    assert c["status"] & oracle_mod.ST_FAULT
    w = S.addr_probe(gaddr, saddr, guard, data, block=32)
    g, _, _, _ = run(oracle_mod, w)
    out = w.output(g, "out")
    assert out[1] == 0 and out[2] == 0
    assert out[0] == g[:4].view("<u4")[0]


# ------------------------------------------------------------------ P11, P12 control flow

def _cfg_case(seed, lanes_data):
    ptx = S.random_cfg_ptx(seed)
    n = len(lanes_data)
    g = np.zeros(8 * n + 4096, np.uint8)
    g[:4 * n] = np.asarray(lanes_data, np.uint32).view(np.uint8)
    params = pack_params([("param_in", "u64", 0), ("param_out", "u64", 4 * n)])
    return ptx, g, params


@pytest.mark.parametrize("seed", range(24))
def test_control_flow_matches_scalar_paths(oracle_mod, seed):
    """Random small CFGs (forward branches, predicated ret) over lanes whose data
    cover every guard pattern: per-lane results equal each lane's own scalar path
    and the thread-instruction total equals the sum of scalar path lengths."""
    rng = np.random.default_rng(seed)
    data = rng.choice([0, 1, 500, 1500, 2500, 2999], size=64)
    ptx, g, params = _cfg_case(seed, data)
    g2 = g.copy()
    c, _, _ = oracle_mod.run(ptx, 1, 64, params, g, trace_cap=256)
    steps = scalar_ref.run_grid(ptx, (1, 1, 1), (64, 1, 1), params, g2)
    assert np.array_equal(g, g2)
    assert int(c["thread_instrs"].sum()) == sum(steps[0])
    assert (c["max_stack_depth"] <= 63).all()


def test_divergence_runs_fall_through_first(oracle_mod):
    """if/else split: the fall-through side issues before the taken side and the
    warp reconverges at the immediate post-dominator with the full mask."""
    ptx = S.HEADER + """.visible .entry d(.param .u64 param_out)
{
    .reg .pred %p<2>;
    .reg .b32 %r<4>;
    .reg .b64 %rd<4>;
    mov.u32 %r1, %laneid;
    setp.lt.u32 %p1, %r1, 16;
    @%p1 bra $L__then;
    add.s32 %r2, %r1, 100;
    bra.uni $L__join;
$L__then:
    add.s32 %r2, %r1, 200;
$L__join:
    ld.param.u64 %rd1, [param_out];
    mul.wide.u32 %rd2, %r1, 4;
    add.s64 %rd3, %rd1, %rd2;
    st.global.u32 [%rd3], %r2;
    ret;
}
"""
    g = np.zeros(256, np.uint8)
    c, t, _ = oracle_mod.run(ptx, 1, 32, pack_params([("param_out", "u64", 0)]), g, trace_cap=32)
    _, rec = oracle_mod.trace_slots(t, 32)
    pcs = rec[0, :c["warp_instrs"][0], 1].tolist()
    assert pcs == [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10]
    out = g[:128].view("<u4")
    assert out.tolist() == [l + 200 if l < 16 else l + 100 for l in range(32)]
    # 3 full + 2 half (else side: lanes 16..31) + 1 half (then side) + 5 full
    assert c["thread_instrs"][0] == 3 * 32 + 2 * 16 + 16 + 5 * 32


def test_random_stress_programs_match_scalar_reference(oracle_mod):
    """Small instances of the random stress generator: SIMT oracle == scalar
    per-thread reference, and thread-instruction totals agree."""
    for seed in range(3):
        nt = 128
        w = W.random_stress(prog_seed=seed, grid=2, block=64, gmem_bytes=1 << 22, n_instr=300, trace_cap=64)
        g, c, _, rc = run(oracle_mod, w, check_races=True)
        assert rc == 0
        g2 = w.gmem.copy()
        steps = scalar_ref.run_grid(w.ptx, w.grid, w.block, w.params_bytes, g2)
        assert np.array_equal(g, g2)
        assert int(c["thread_instrs"].sum()) == sum(sum(s) for s in steps)
        assert nt == 128


# ------------------------------------------------------------------ P13 post-dominators

def _brute_ipdom(prog):
    n = len(prog.code)
    EXIT = n
    succ = []
    for i, (guard, parts, ops) in enumerate(prog.code):
        nx = i + 1
        if parts[0] == "bra":
            t = prog.labels[ops[0]]
            s = {t}
            if guard is not None:
                s.add(nx)
        elif parts[0] in ("ret", "exit"):
            s = {EXIT}
            if guard is not None:
                s.add(nx)
        else:
            s = {nx}
        succ.append({EXIT if x >= n else x for x in s})

    def reaches_exit(v, removed):
        seen, stack = set(), [v]
        while stack:
            x = stack.pop()
            if x == EXIT:
                return True
            if x in seen or x == removed:
                continue
            seen.add(x)
            stack.extend(succ[x])
        return False

    out = []
    for v, (guard, parts, ops) in enumerate(prog.code):
        if parts[0] != "bra" or guard is None:
            out.append(0xFFFFFFFF)
            continue
        if not reaches_exit(v, None):
            out.append(n)
            continue
        strict = [d for d in range(n) if d != v and not reaches_exit(v, d)]
        best = n
        for d in strict:
            if all(d2 == d or not reaches_exit(d, d2) for d2 in strict):
                best = d
        out.append(best)
    return out


@pytest.mark.parametrize("seed", range(40))
def test_ipdom_matches_brute_force(oracle_mod, seed):
    ptx = S.random_cfg_ptx(1000 + seed, n_instr=16, loops=(seed % 2 == 1))
    got = oracle_mod.ipdom_table(ptx)
    exp = _brute_ipdom(scalar_ref.Program(ptx))
    assert got == exp


# ------------------------------------------------------------------ P14 trace slots, P15 stack

def test_trace_slot_layout_and_overflow(oracle_mod):
    w = W.ffma_probe(n_acc=8, iters=4, grid=1, block=64, trace_cap=50)
    _, c, t, _ = run(oracle_mod, w)
    assert t.size == 2 * (16 + 8 * 50)
    hdr, rec = oracle_mod.trace_slots(t, 50)
    for k in range(2):
        n = int(c["warp_instrs"][k])
        assert n > 50
        assert hdr[k]["records_written"] == 50
        assert hdr[k]["records_written"] + hdr[k]["records_dropped"] == n
        assert hdr[k]["flags"] & 1 and c["status"][k] & oracle_mod.ST_TRACE_DROP
        cyc = rec[k, :, 0].astype(np.int64)
        assert (np.diff(cyc) >= 1).all()
    # cap 0: header only
    _, c0, t0, _ = run(oracle_mod, w, trace_cap=0)
    h0, _ = oracle_mod.trace_slots(t0, 0)
    assert t0.size == 32 and (h0["records_written"] == 0).all()
    assert (h0["records_dropped"] == c0["warp_instrs"]).all()


def test_stack_depth_bound_is_reached_exactly(oracle_mod):
    ptx = S.staircase_ptx(31)
    g = np.zeros(256, np.uint8)
    c, _, _ = oracle_mod.run(ptx, 1, 32, pack_params([("param_out", "u64", 0)]), g, trace_cap=8)
    assert c["max_stack_depth"][0] == 63 and c["diverge_n"][0] == 31
    out = g[:128].view("<u4").tolist()
    assert out == [2 * (k + 1) for k in range(31)] + [1031]


# ------------------------------------------------------------------ status and error paths

def test_parse_errors_carry_line_numbers(oracle_mod):
    bad = W.VECTOR_ADD_PTX.replace("add.f32 %f3, %f1, %f2;", "add.f32 %f3, %f1, %f9;")
    with pytest.raises(oracle_mod.OracleError) as e:
        oracle_mod.program_info(bad)
    line = 1 + W.VECTOR_ADD_PTX.split("add.f32 %f3")[0].count("\n")
    assert ("line %d:" % line) in str(e.value) and "%f9" in str(e.value)
    with pytest.raises(oracle_mod.OracleError) as e:
        oracle_mod.program_info(W.VECTOR_ADD_PTX.replace("add.f32 %f3", "div.rn.f32 %f3"))
    assert e.value.code == -2
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.program_info(W.VECTOR_ADD_PTX.replace("$L__exit;", "$L__nowhere;"))
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.program_info(W.VECTOR_ADD_PTX.replace("mov.u32 %r2, %tid.x;", "mov.u32 %r2, 1.5;"))


def test_budget_stops_warps(oracle_mod):
    w = W.vector_add()
    g, c, t, _ = run(oracle_mod, w, max_warp_instrs=10)
    assert (c["warp_instrs"] == 10).all()
    assert (c["status"] & oracle_mod.ST_BUDGET).all() and not (c["status"] & oracle_mod.ST_FINISHED).any()
    assert (w.output(g, "c") == 0).all()


def test_barrier_in_divergent_region_is_flagged(oracle_mod):
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
    g = np.zeros(64, np.uint8)
    c, _, _ = oracle_mod.run(ptx, 1, 64, pack_params([("param_out", "u64", 0)]), g, trace_cap=8)
    assert (c["status"] & oracle_mod.ST_BARDIV).all()
    assert (c["status"] & oracle_mod.ST_FINISHED).all()
    assert (c["barrier_n"] == 1).all()


def test_cycle_overflow_stops_warp(oracle_mod):
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
    g = np.zeros(64, np.uint8)
    lat = oracle_mod.default_latency()
    lat[7] = 65535  # ld.global
    c, _, _ = oracle_mod.run(ptx, 1, 32, pack_params([("param_out", "u64", 0)]), g, trace_cap=4, latency=lat)
    assert c["status"][0] & oracle_mod.ST_CYCLE_OVF
    assert c["cycles"][0] <= 0x80000000


def test_race_checker(oracle_mod):
    for s in (1, 3):
        w = W.bank_probe(s, iters=2, grid=1, block=128, trace_cap=4)
        _, _, _, rc = run(oracle_mod, w, check_races=True)
        assert rc == 0
    racy = S.HEADER + """.visible .entry r(.param .u64 param_out)
{
    .reg .b32 %r<3>;
    .reg .b64 %rd<2>;
    ld.param.u64 %rd1, [param_out];
    mov.u32 %r1, %laneid;
    st.global.u32 [%rd1], %r1;
    ret;
}
"""
    g = np.zeros(64, np.uint8)
    _, _, rc = oracle_mod.run(racy, 1, 32, pack_params([("param_out", "u64", 0)]), g, check_races=True)
    assert rc == oracle_mod.E_RACE
    # lane-ascending order: the highest lane's store is the one that remains
    assert g[:4].view("<u4")[0] == 31


RW_PTX = S.HEADER + """.visible .entry rw(.param .u64 param_out, .param .u32 param_wb, .param .u32 param_val)
{
    .reg .pred %p<2>;
    .reg .b32 %r<6>;
    .reg .b64 %rd<4>;
    ld.param.u64 %rd1, [param_out];
    ld.param.u32 %r1, [param_wb];
    ld.param.u32 %r2, [param_val];
    mov.u32 %r3, %tid.x;
    mov.u32 %r4, %ctaid.x;
    mul.wide.u32 %rd2, %r3, 4;
    add.s64 %rd3, %rd1, %rd2;
    setp.ne.u32 %p1, %r4, %r1;
    @%p1 bra $L__read;
    st.global.u32 [%rd3], %r2;
$L__read:
    ld.global.u32 %r5, [%rd3];
    ret;
}
"""


@pytest.mark.parametrize("grid,writer,val,racy", [
    (2, 0, 7, True),    # the other block reads after the write in simulation order
    (2, 1, 7, True),    # ... and before it
    (2, 0, 0, False),   # the write stores the value the word already holds
    (1, 0, 7, False),   # each thread reads back only its own write
])
def test_race_checker_independent_of_simulation_order(oracle_mod, grid, writer, val, racy):
    """Block `writer` stores `val` to word tid and every thread then loads word tid.
    A load by a thread of another block could see the word before or after the
    store, whichever block runs first, unless the store leaves the word unchanged:
    the checker must flag it in both simulation orders, and only then."""
    g = np.zeros(4096, np.uint8)
    pb = pack_params([("param_out", "u64", 0), ("param_wb", "u32", writer), ("param_val", "u32", val)])
    _, _, rc = oracle_mod.run(RW_PTX, grid, 64, pb, g, check_races=True)
    assert rc == (oracle_mod.E_RACE if racy else 0)
    assert (g[:256].view("<u4") == val).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_stress_full_programs_are_race_free(oracle_mod, seed):
    """The 2000-instruction stress programs (the parity set, seeds 0-2) at 64 x 256
    threads: the race checker finds no byte that two threads access with an
    order-dependent outcome (two writes of different values, or a read and a write
    of another value), over the whole run for global memory and within one barrier
    interval for shared memory, so results do not depend on the order warps run in."""
    w = W.random_stress(prog_seed=seed, grid=64, gmem_bytes=1 << 26)
    _, c, _, rc = run(oracle_mod, w, trace_cap=4, check_races=True, threads=8)
    assert rc == 0
    assert (c["status"] & oracle_mod.ST_FINISHED).all()
    assert int(c["barrier_n"].max()) > 50 and int(c["gst_n"].sum()) > 0


def test_block_subset_equals_full_run(oracle_mod):
    w = W.strided_gather(2, n=4096)
    g_full, c_full, t_full, _ = run(oracle_mod, w)
    blocks = [3, 0, 15]
    g_sub, c_sub, t_sub, _ = run(oracle_mod, w, blocks=blocks)
    wpb = w.warps_per_block
    for i, b in enumerate(blocks):
        assert np.array_equal(c_sub[i * wpb:(i + 1) * wpb], c_full[b * wpb:(b + 1) * wpb])
    out_full, out_sub = w.output(g_full, "c"), w.output(g_sub, "c")
    for b in blocks:
        assert np.array_equal(out_sub[b * 256:(b + 1) * 256], out_full[b * 256:(b + 1) * 256])


def test_thread_count_does_not_change_results(oracle_mod):
    w = W.random_stress(prog_seed=1, grid=16, block=64, gmem_bytes=1 << 22, n_instr=200, trace_cap=64)
    g1, c1, t1, _ = run(oracle_mod, w, threads=1)
    g8, c8, t8, _ = run(oracle_mod, w, threads=8)
    assert np.array_equal(g1, g8) and np.array_equal(c1, c8) and np.array_equal(t1, t8)


def test_single_ret_program(oracle_mod):
    """The smallest program, a lone ret, on 33-thread blocks (a full warp and a
    one-lane warp): each warp issues once, at cycle 0, with its live lanes, then
    finishes; cycles = last issue + 1 = 1, stack depth 1, nothing else counted."""
    ptx = S.HEADER + ".visible .entry k()\n{\n    ret;\n}\n"
    co, to, _ = oracle_mod.run(ptx, (3, 1, 1), (33, 1, 1), b"", np.zeros(64, np.uint8), trace_cap=4)
    assert list(co["thread_instrs"]) == [32, 1] * 3
    assert (co["warp_instrs"] == 1).all() and (co["cycles"] == 1).all() and (co["stall_cycles"] == 0).all()
    assert (co["status"] == 1).all() and (co["max_stack_depth"] == 1).all()
    for f in ("gld_n", "gst_n", "sh_n", "diverge_n", "barrier_n", "fault_n"):
        assert (co[f] == 0).all(), f
    hs, rs = oracle_mod.trace_slots(to, 4)
    assert (hs["records_written"] == 1).all() and list(hs["warp_in_block"]) == [0, 1] * 3
    assert (rs[:, 0] == 0).all()  # issue cycle 0, pc 0
    assert (hs["flags"] == 8).all()  # finished
    # a budget of 0 stops every warp before its one issue: status and flag BUDGET, nothing written
    co, to, _ = oracle_mod.run(ptx, (3, 1, 1), (33, 1, 1), b"", np.zeros(64, np.uint8), trace_cap=4, max_warp_instrs=0)
    hs, _ = oracle_mod.trace_slots(to, 4)
    assert (co["status"] == 2).all() and (co["warp_instrs"] == 0).all() and (co["cycles"] == 0).all()
    assert (hs["flags"] == 4).all() and (hs["records_written"] == 0).all()


def test_largest_shared_window_edges(oracle_mod):
    """The 65536-byte shared window at its edges (workloads.small.shared_edges_ptx):
    values written before a barrier by other warps are read back at the first and
    last KiB, the last word and the last 8 bytes as one 64-bit load; the word just
    past the end and a misaligned word fault and read 0 (fault_n 2 x 32 per warp);
    every access is stride 1 or a broadcast, so each has bank degree 1."""
    import struct
    g = np.zeros(2 * 256 * 32, np.uint8)
    co, to, _ = oracle_mod.run(S.shared_edges_ptx(), (2, 1, 1), (256, 1, 1), struct.pack("<Q", 0), g, trace_cap=64)
    hs, _ = oracle_mod.trace_slots(to, 64)
    assert (hs["flags"] == 2 | 8).all()  # fault, finished
    out = g.view(np.uint32).reshape(512, 8)
    t = np.arange(512) % 256
    nb = np.where(t == 255, 0, t + 1)
    assert (out[:, 0] == nb + 1).all() and (out[:, 1] == nb + 7).all() and (out[:, 2] == 262).all()
    assert (out[:, 3] == 0).all() and (out[:, 4] == 0).all() and (out[:, 5] == 0).all()
    assert (out[:, 6] == 261).all() and (out[:, 7] == 262).all()
    assert (co["fault_n"] == 64).all() and (co["sh_n"] == 8).all()
    assert (co["sh_degree_sum"] == 8).all() and (co["sh_degree_max"] == 1).all()
    assert (co["status"] == 5).all()  # finished, fault


def test_latency_class_of_every_producer(oracle_mod):
    """Each producer of workloads.small.LATENCY_PAIRS (every destination-writing
    form of the subset) is followed by a consumer of its result: as an operand,
    a guard, a store's value or address, or a load's address.  With a latency
    table of distinct values (101 + 10 k for class k), a producer issues one cycle
    after the previous consumer (its sources are long ready) and its consumer
    exactly its class's latency later, so a form put in the wrong class fails."""
    import struct
    lat = [101 + 10 * k for k in range(14)] + [28, 150, 400, 0]
    g = np.zeros(4096, np.uint8)
    co, to, _ = oracle_mod.run(S.latency_classes_ptx(), (1, 1, 1), (32, 1, 1), struct.pack("<QI", 64, 0), g,
                               trace_cap=128, latency=lat)
    hs, rs = oracle_mod.trace_slots(to, 128)
    iss = rs[0, :int(hs["records_written"][0]), 0].astype(np.int64)
    assert co["status"][0] == 1 and co["fault_n"][0] == 0
    first = 12  # the prologue's six producer/consumer pairs
    for k, (prod, cls, _) in enumerate(S.LATENCY_PAIRS):
        i = first + 2 * k
        assert iss[i] - iss[i - 1] == 1, prod
        assert iss[i + 1] - iss[i] == lat[oracle_mod.LAT_NAMES.index(cls)], (prod, cls)
    assert len(iss) == first + 2 * len(S.LATENCY_PAIRS) + 1  # and the ret


@pytest.mark.parametrize("block", [64, 256, 1024])
def test_block_reduce_closed_form(oracle_mod, block):
    """The shared-memory tree reduction (workloads.small.block_reduce_ptx): each
    block's output is the wrapping sum of its inputs; only warp 0 diverges, at the
    five steps with s < 32 and at the final t == 0 branch; every thread passes
    1 + log2(block) barriers; every shared access has bank degree 1 (stride 1)."""
    import struct
    grid = 8
    data = np.random.default_rng(11).integers(0, 1 << 32, size=grid * block, dtype=np.uint32)
    out = 4 * grid * block
    g = np.zeros(out + 4 * grid, np.uint8)
    g[:out] = data.view(np.uint8)
    co, _, _ = oracle_mod.run(S.block_reduce_ptx(block), (grid, 1, 1), (block, 1, 1), struct.pack("<QQ", 0, out), g,
                              trace_cap=0)
    exp = (data.reshape(grid, block).astype(np.uint64).sum(axis=1) % (1 << 32)).astype(np.uint32)
    assert np.array_equal(g[out:].view(np.uint32), exp)
    wpb = block // 32
    warp0 = (np.arange(len(co)) % wpb) == 0
    assert (co["diverge_n"][warp0] == 6).all() and (co["diverge_n"][~warp0] == 0).all()
    assert (co["barrier_n"] == 1 + int(np.log2(block))).all()
    assert (co["sh_degree_max"] == 1).all() and (co["fault_n"] == 0).all()


@pytest.mark.parametrize("pad", [0, 1])
def test_tile_transpose_closed_form(oracle_mod, pad):
    """The shared-tile transpose (workloads.small.tile_transpose_ptx): out is the
    exact transpose; the tile's row store is stride 1 (degree 1) and its column
    load is stride 32 + pad words, degree 32 without padding and 1 with it; both
    global sides stay coalesced (4 sectors, 1 line per warp access)."""
    import struct
    gx = 3
    n = 32 * gx
    data = np.random.default_rng(5).integers(0, 1 << 32, size=n * n, dtype=np.uint32)
    g = np.zeros(8 * n * n, np.uint8)
    g[:4 * n * n] = data.view(np.uint8)
    co, _, _ = oracle_mod.run(S.tile_transpose_ptx(pad), (gx, gx, 1), (32, 32, 1),
                              struct.pack("<QQ", 0, 4 * n * n), g, trace_cap=0)
    assert np.array_equal(g[4 * n * n:].view(np.uint32).reshape(n, n), data.reshape(n, n).T)
    assert (co["sh_n"] == 2).all()
    assert (co["sh_degree_max"] == (32 if pad == 0 else 1)).all()
    assert (co["sh_degree_sum"] == (33 if pad == 0 else 2)).all()
    for f in ("gld_sectors", "gst_sectors"):
        assert (co[f] == 4).all(), f
    assert (co["gld_lines"] == 1).all() and (co["gst_lines"] == 1).all()


def test_stencil3_closed_form(oracle_mod):
    """The 3-point stencil (workloads.small.stencil3_ptx) over n = 1000 on 128-thread
    blocks: out = in[i-1] + in[i] + in[i+1] inside, in[i] at the ends.  An interior
    warp's three loads cover 4 + 5 + 5 sectors and 1 + 2 + 2 lines (the shifted
    loads straddle a 128-byte line), its store 4 sectors in 1 line; warp 0 leaves
    lane 0 out of the shifted loads (13 sectors, 4 lines, one divergence); the last
    warp, with 8 live threads of which the last is an end, counts 4 sectors, 4 lines
    and two divergences."""
    import struct
    n, block = 1000, 128
    data = np.random.default_rng(3).integers(0, 1 << 32, size=n, dtype=np.uint32)
    off = 8192
    g = np.zeros(off + 4 * n, np.uint8)
    g[:4 * n] = data.view(np.uint8)
    co, _, _ = oracle_mod.run(S.stencil3_ptx(), ((n + block - 1) // block, 1, 1), (block, 1, 1),
                              struct.pack("<QQI", 0, off, n), g, trace_cap=0)
    d = data.astype(np.uint64)
    exp = d.copy()
    exp[1:-1] = (d[:-2] + d[1:-1] + d[2:]) % (1 << 32)
    assert np.array_equal(g[off:].view(np.uint32), exp.astype(np.uint32))
    row = lambda k: tuple(int(co[f][k]) for f in ("gld_n", "gld_sectors", "gld_lines", "gst_n", "gst_sectors",
                                                  "gst_lines", "diverge_n"))
    assert row(0) == (3, 13, 4, 1, 4, 1, 1)
    assert all(row(k) == (3, 14, 5, 1, 4, 1, 0) for k in range(1, 31))
    assert row(31) == (3, 4, 4, 1, 1, 1, 2)


def test_lcg64_against_numpy(oracle_mod):
    """64-bit integer forms (workloads.small.lcg64_ptx): mad.lo.u64 iterated in a
    loop, mul.lo/add/sub.u64, unsigned and signed 64-bit setp, selp.b64 and u64
    loads and stores equal numpy's wrapping uint64 arithmetic; the signed and
    unsigned compares disagree on part of the threads, so both are exercised."""
    import struct
    nt, block = 512, 128
    seeds = np.random.default_rng(9).integers(0, 1 << 63, size=nt, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    so, oo, fo = 0, 8 * nt, 32 * nt
    g = np.zeros(fo + 4 * nt, np.uint8)
    g[:8 * nt] = seeds.view(np.uint8)
    oracle_mod.run(S.lcg64_ptx(), (nt // block, 1, 1), (block, 1, 1), struct.pack("<QQQ", so, oo, fo), g, trace_cap=0)
    a, c = np.uint64(6364136223846793005), np.uint64(1442695040888963407)
    with np.errstate(over="ignore"):
        x = seeds.copy()
        for _ in range(37):
            x = x * a + c
        y = x * x + x - c
    out = g[oo:fo].view(np.uint64).reshape(nt, 3)
    assert np.array_equal(out[:, 0], x) and np.array_equal(out[:, 1], y)
    assert np.array_equal(out[:, 2], np.where(x < y, x, y))
    s = (x.view(np.int64) < y.view(np.int64)).astype(np.uint32)
    assert np.array_equal(g[fo:].view(np.uint32), s)
    assert (s != (x < y)).any()


def test_extra_workloads_are_race_free(oracle_mod):
    """The race checker passes the reduction, transpose, stencil, 64-bit and
    shared-edge programs at the shapes their tests use, and catches the 64-bit
    program on a grid larger than its arrays (its extra threads write the flags of
    others: the case the GPU parity test must avoid).  (The latency-class program
    has every thread store one and the same value to one shared word, a race the
    checker reports but whose result cannot depend on the order.)"""
    import struct
    z = lambda n: np.zeros(n, np.uint8)
    cases = [
        (S.block_reduce_ptx(256), (4, 1, 1), (256, 1, 1), struct.pack("<QQ", 0, 4096), z(4096 + 16)),
        (S.tile_transpose_ptx(0), (2, 2, 1), (32, 32, 1), struct.pack("<QQ", 0, 16384), z(32768)),
        (S.tile_transpose_ptx(1), (2, 2, 1), (32, 32, 1), struct.pack("<QQ", 0, 16384), z(32768)),
        (S.stencil3_ptx(), (4, 1, 1), (128, 1, 1), struct.pack("<QQI", 0, 4096, 500), z(8192)),
        (S.lcg64_ptx(4), (2, 1, 1), (160, 1, 1), struct.pack("<QQQ", 0, 2560, 10240), z(10240 + 1280)),
        (S.shared_edges_ptx(), (1, 1, 1), (256, 1, 1), struct.pack("<Q", 0), z(8192)),
    ]
    for ptx, grid, block, params, g in cases:
        _, _, rc = oracle_mod.run(ptx, grid, block, params, g, check_races=True)
        assert rc == 0, ptx.split("(")[0][-40:]
    # 300 threads' arrays on a 320-thread grid: threads 300..319 write over flags 0..119
    nt = 300
    g = z(32 * nt + 4 * nt)
    _, _, rc = oracle_mod.run(S.lcg64_ptx(4), (2, 1, 1), (160, 1, 1), struct.pack("<QQQ", 0, 8 * nt, 32 * nt), g,
                              check_races=True)
    assert rc == oracle_mod.E_RACE


def test_setp_forms_against_numpy(oracle_mod):
    """The unsigned setp mnemonics (lo ls hi hs), eq/ne on .b32 and .b64, 64-bit
    unsigned compares and the .u32 forms of mul.lo and mad.lo, one flag bit per
    comparison (workloads.small.setp_forms_ptx), against numpy over inputs with
    equal and adjacent pairs; every bit is set for some threads and clear for others."""
    import struct
    nt = 1024
    a, b, c, d, offs, g = S.setp_forms_inputs(nt, 4)
    oracle_mod.run(S.setp_forms_ptx(), (nt // 256, 1, 1), (256, 1, 1), struct.pack("<5Q", *offs), g, trace_cap=0)
    out = offs[4]
    sa, sb = a.view(np.int32), b.view(np.int32)
    bits = [a < b, a <= b, a > b, a >= b, a == b, a != b, c < d, c >= d, c == d, c != d, sa <= sb, a >= b]
    assert len(bits) == len(S.SETP_FORMS)
    exp = sum(e.astype(np.uint32) << k for k, e in enumerate(bits)).astype(np.uint32)
    assert np.array_equal(g[out:out + 4 * nt].view(np.uint32), exp)
    assert all(0 < e.mean() < 1 for e in bits)
    with np.errstate(over="ignore"):
        assert np.array_equal(g[out + 65536:out + 65536 + 4 * nt].view(np.uint32), a * b)
        assert np.array_equal(g[out + 131072:out + 131072 + 4 * nt].view(np.uint32), a * b + a)


def test_f32_setp_against_numpy(oracle_mod):
    """setp.{eq,ne,lt,le,gt,ge}.f32 and selp.f32 (workloads.small.f32_setp_ptx) over
    the edge-value crossing (NaN, +-0, +-inf, subnormals, extremes) and random
    patterns, against numpy's comparisons with the ordered reading: every
    comparison, ne included, is false when an operand is NaN; +0 == -0."""
    import struct
    ops = S.f32_operands(4096, 7)[:, :2].copy()
    n = len(ops)
    out = 8 * n + 4096
    g = np.zeros(out + 65536 + 4 * n, np.uint8)
    g[:8 * n] = ops.reshape(-1).view(np.uint8)
    oracle_mod.run(S.f32_setp_ptx(), ((n + 255) // 256, 1, 1), (256, 1, 1), struct.pack("<QQI", 0, out, n), g,
                   trace_cap=0)
    a, b = ops[:, 0].view(np.float32), ops[:, 1].view(np.float32)
    nan = np.isnan(a) | np.isnan(b)
    assert nan.any() and ((a == 0) & (b == 0) & (ops[:, 0] != ops[:, 1])).any()  # NaNs and +0 vs -0 occur
    with np.errstate(invalid="ignore"):
        bits = [a == b, (a != b) & ~nan, a < b, a <= b, a > b, a >= b]
        pick = np.where(a < b, ops[:, 0], ops[:, 1])
    exp = sum(e.astype(np.uint32) << k for k, e in enumerate(bits)).astype(np.uint32)
    assert np.array_equal(g[out:out + 4 * n].view(np.uint32), exp)
    assert np.array_equal(g[out + 65536:out + 65536 + 4 * n].view(np.uint32), pick)
