"""GPU: the simulated probe suite (SASS-probe method, sections 12-15).

Each probe program runs through the C ABI on gfx950 and must match the CPU
oracle bit for bit (memory, every counter); the probe-suite analysis computed
from the GPU's counters must then give the closed forms that the CPU pins
(tests/test_probe_pins.py) derive by hand from the issue rule.
"""
import numpy as np
import pytest

from workloads import probes as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from analysis_ptxsimulator_amd import ks
    ks.lib()
    return ks


@pytest.fixture(scope="module")
def PS(K):
    from analysis_ptxsimulator_amd import probes
    return probes


def _say(msg):
    print("[gpu] " + msg, flush=True)


@pytest.mark.parametrize("op", list(P.OPS))
@pytest.mark.parametrize("k", [1, 3, 8])
def test_probe_parity(K, oracle_mod, op, k):
    w = P.chain_probe(op, k, iters=6, grid=3, block=96, trace_cap=64)
    _say("%s grid=%s block=%s" % (w.name, w.grid, w.block))
    s = K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=w.trace_cap)
    try:
        s.load_gmem(w.gmem)
        s.run(w.params_bytes)
        gg, cg, tg = s.read_gmem(), s.read_counters(), s.read_trace()
    finally:
        s.close()
    go = w.gmem.copy()
    co, to, _ = oracle_mod.run(w.ptx, w.grid, w.block, w.params_bytes, go, trace_cap=w.trace_cap)
    assert np.array_equal(gg, go)
    for f in co.dtype.names:
        assert np.array_equal(cg[f], co[f]), f
    hg, rg = K.trace_slots(tg, w.trace_cap)
    ho, ro = K.trace_slots(to, w.trace_cap)
    assert np.array_equal(hg, ho)
    for i in range(len(ho)):
        n = int(ho["records_written"][i])
        assert np.array_equal(rg[i, :n], ro[i, :n]), i


def test_suite_controls_and_accumulators(PS):
    _say("probe suite: controls, accumulator sweep")
    rows = {r["op"]: r for r in PS.control_suite()}
    assert rows["none"]["cycles_per_iteration"] == 9
    for op in ("fma.f32", "add.s32", "add.f32"):
        assert rows[op]["cycles_per_iteration"] == 128
        assert rows[op]["corrected_cycles_per_iteration"] == 119
    acc = PS.accumulator_sweep()
    assert [r["cycles_per_instruction"] for r in acc] == [4.0, 2.0, 35 / 32, 35 / 32, 35 / 32]
    # each extra accumulator is one more declared register slot
    slots = [r["register_slots"] for r in acc]
    assert [b - a for a, b in zip(slots, slots[1:])] == [b - a for a, b in zip(P.ACC_SWEEP, P.ACC_SWEEP[1:])]


def test_suite_count_sweep(PS):
    _say("probe suite: count sweep")
    for k, per_target in ((1, 4.0), (8, 35 / 32)):
        r = PS.count_sweep("fma.f32", k)
        assert r["r2"] == pytest.approx(1.0, abs=1e-12)
        assert r["slope"] == pytest.approx(per_target, rel=1e-12)
        d = np.diff(r["cycles"]) / np.diff(r["N"])
        assert np.all(d == per_target)
    # another latency table: the slope follows the table (dependent chain: L cycles per target)
    lat = [4] * 16
    lat[2], lat[7], lat[8], lat[9], lat[10], lat[12] = 6, 200, 23, 200, 23, 20
    r = PS.count_sweep("fma.f32", 1, iters=(16, 64, 256), latency=lat)
    assert r["slope"] == pytest.approx(6.0, rel=1e-12)


def test_suite_warp_sweep(PS):
    _say("probe suite: warp sweep")
    rows = PS.warp_sweep()
    one = rows[0]
    for r in rows:
        assert r["warps"] == r["blocks"] * ((r["threads"] + 31) // 32)
        assert r["cycles_per_instruction"] == one["cycles_per_instruction"]
        assert r["instructions_per_cycle"] == pytest.approx(r["warps"] * one["instructions_per_cycle"], rel=1e-12)
        assert r["gpu_ms"] > 0
