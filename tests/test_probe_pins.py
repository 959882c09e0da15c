"""Pins of the probe programs on the CPU oracle (SASS-probe method, sections 12-15).

Every expected number below is derived by hand from the issue rule of the
KernelScope latency model as this simulator reads it (an instruction issues at
the later of the previous issue + 1 and the ready cycle of its sources; a
destination is ready `latency` cycles after issue) and from the probe's loop
layout (counter add, 16 targets, setp, 16 targets, @p bra):

* one accumulator: every target waits for the previous one, the setp and the bra
  fill the shadows, so an iteration costs 32 L (L >= 3);
* two accumulators: the targets pair up, an iteration costs 16 L (L >= 4);
* at least L accumulators: nothing waits, the 35 instructions of an iteration
  issue back to back: 35 cycles;
* the empty loop: add -> setp -> bra -> next add, L_int32 + L_setp + 1 cycles.

The per-thread outputs are pinned by arithmetic that the simulator does not
share: integer chains in closed form modulo 2^32, f32 add and mul chains by
numpy's float32 (IEEE round-to-nearest) evaluated step by step, and the f32 FMA
chain by the exact rational rounding of tests/ieee32.py.
"""
import numpy as np
import pytest

from workloads import probes as P
from tests import ieee32

INT32, SETP, FP32 = 0, 3, 2


def lat_table(oracle_mod, fp32=4, int32=4, setp=4):
    lat = oracle_mod.default_latency()
    lat[FP32], lat[INT32], lat[SETP] = fp32, int32, setp
    return lat


def run(oracle_mod, w, lat=None):
    g = w.gmem.copy()
    c, _, _ = oracle_mod.run(w.ptx, w.grid, w.block, w.params_bytes, g, trace_cap=0, latency=lat)
    return c, g


def per_iter(oracle_mod, op, k, lat=None, iters=(8, 13)):
    t = [int(run(oracle_mod, P.chain_probe(op, k, i), lat)[0]["cycles"][0]) for i in iters]
    return (t[1] - t[0]) / (iters[1] - iters[0])


def op_latency(op, fp32, int32):
    return fp32 if P.OP_LATENCY_CLASS[op] == "fp32" else int32


@pytest.mark.parametrize("op", [o for o in P.OPS if o != "none"])
@pytest.mark.parametrize("fp32,int32", [(4, 4), (6, 5), (3, 7)])
def test_dependent_and_independent_chains(oracle_mod, op, fp32, int32):
    lat = lat_table(oracle_mod, fp32, int32)
    L = op_latency(op, fp32, int32)
    assert per_iter(oracle_mod, op, 1, lat) == 32 * L
    if L >= 4:
        assert per_iter(oracle_mod, op, 2, lat) == 16 * L
    for k in (8, 16):
        if k >= L:
            assert per_iter(oracle_mod, op, k, lat) == 35


@pytest.mark.parametrize("int32,setp", [(4, 4), (5, 2), (9, 1)])
def test_empty_loop_control(oracle_mod, int32, setp):
    lat = lat_table(oracle_mod, int32=int32, setp=setp)
    assert per_iter(oracle_mod, "none", 1, lat) == int32 + setp + 1
    # corrected cost of the dependent FMA chain = probe - empty loop (section 12.2)
    assert per_iter(oracle_mod, "fma.f32", 1, lat) - per_iter(oracle_mod, "none", 1, lat) == 32 * 4 - (int32 + setp + 1)


def test_count_sweep_is_exactly_affine(oracle_mod):
    """Section 13: T(N) = L N + C with R^2 = 1: every iteration adds the same cycles."""
    for k, slope in ((1, 128), (8, 35)):
        its = (1, 2, 5, 17, 64)
        T = [int(run(oracle_mod, P.chain_probe("fma.f32", k, i))[0]["cycles"][0]) for i in its]
        C = T[0] - slope
        assert T == [slope * i + C for i in its]


def test_accumulator_sweep_shape(oracle_mod):
    """Section 14: cycles per target instruction 4, 2, then the issue bound 35/32
    (the page's hardware numbers: 4.00, 2.02, 1.03, 1.01, 1.02)."""
    cpi = [per_iter(oracle_mod, "fma.f32", k) / 32 for k in P.ACC_SWEEP]
    assert cpi == [4.0, 2.0, 35 / 32, 35 / 32, 35 / 32]


def test_warp_sweep_warps_are_independent(oracle_mod):
    """Section 15: every warp of every launch shape runs the same simulated cycles
    as a single warp (no shared issue resources in this model)."""
    c1, _ = run(oracle_mod, P.chain_probe("fma.f32", 1, 16, grid=1, block=1))
    for grid, block in ((1, 32), (1, 64), (1, 128), (3, 128)):
        c, _ = run(oracle_mod, P.chain_probe("fma.f32", 1, 16, grid=grid, block=block))
        assert len(c) == grid * ((block + 31) // 32)
        assert (c["cycles"] == c1["cycles"][0]).all()
        assert (c["warp_instrs"] == c1["warp_instrs"][0]).all()
        assert int(c["thread_instrs"].sum()) == grid * block * int(c1["warp_instrs"][0])


@pytest.mark.parametrize("k", [1, 3, 8])
def test_integer_chain_outputs(oracle_mod, k):
    iters = 5
    n = 32 * iters
    for op in ("add.s32", "mul.s32", "mad.s32"):
        w = P.chain_probe(op, k, iters, grid=2, block=48)
        _, g = run(oracle_mod, w)
        nt = 2 * 48
        x = w.gmem[0: 4 * nt].view("<u4").astype(object)
        off_y = w.params[1][2]
        off_o = w.params[2][2]
        y = w.gmem[off_y: off_y + 4 * nt].view("<u4").astype(object)
        out = g[off_o: off_o + 4 * nt].view("<u4")
        M = 1 << 32
        per_acc = [len(range(j, 32, k)) * iters for j in range(k)]  # updates of each accumulator
        for t in range(nt):
            if op == "add.s32":
                want = sum(p * x[t] for p in per_acc) % M
            elif op == "mad.s32":
                want = sum(p * x[t] * y[t] for p in per_acc) % M
            else:
                want = sum(pow(int(x[t]), p, M) for p in per_acc) % M
            assert int(out[t]) == want, (op, k, t)
        assert n == sum(per_acc)


@pytest.mark.parametrize("op", ["add.f32", "mul.f32"])
def test_f32_add_mul_chain_outputs(oracle_mod, op):
    iters, k = 3, 2
    w = P.chain_probe(op, k, iters, grid=1, block=32)
    _, g = run(oracle_mod, w)
    x = w.gmem[0:128].view("<f4")
    off_o = w.params[2][2]
    out = g[off_o: off_o + 128].view("<u4")
    for t in range(32):
        acc = [np.float32(0.0 if op == "add.f32" else 1.0) for _ in range(k)]
        for _ in range(iters):
            for j in range(32):
                acc[j % k] = np.float32(acc[j % k] + x[t]) if op == "add.f32" else np.float32(acc[j % k] * x[t])
        s = acc[0]
        for a in acc[1:]:
            s = np.float32(s + a)
        assert int(out[t]) == int(np.float32(s).view(np.uint32)), t


def test_fma_chain_output_exact(oracle_mod):
    iters, k = 2, 1
    w = P.chain_probe("fma.f32", k, iters, grid=1, block=32)
    _, g = run(oracle_mod, w)
    off_y, off_o = w.params[1][2], w.params[2][2]
    x = w.gmem[0:128].view("<u4")
    y = w.gmem[off_y: off_y + 128].view("<u4")
    out = g[off_o: off_o + 128].view("<u4")
    for t in range(0, 32, 5):
        acc = 0
        for _ in range(32 * iters):
            acc = ieee32.fma(int(x[t]), int(y[t]), acc)
        assert int(out[t]) == acc, t
