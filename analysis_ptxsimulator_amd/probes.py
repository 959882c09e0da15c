"""The SASS-probe method, run inside the simulator on the GPU.

The SASS-probe method page (teach-meaning.tistory.com/1954) measures hardware
instruction latency with probe loops and controls the measurement in several
ways.  Here the probe programs (workloads/probes.py) run through libkscope's
interpreter, and the same controls are computed from the simulated per-warp
cycle counters instead of clock reads:

* control experiments (section 12): the empty loop, and dependent chains of
  other instruction kinds; corrected cycles = probe - empty loop (12.2);
* instruction-count sweep (section 13): T(N) fitted to L * N + C by least
  squares, with slope, intercept and R^2;
* accumulator sweep (section 14): cycles per target instruction for 1, 2, 4, 8
  and 16 independent accumulators, with the register slots the probe declares
  (the simulator has no register allocator, so nothing ever spills);
* warp-count sweep (section 15): the same probe on more warps, with the
  instructions per simulated cycle of the whole launch.

Every simulated number is a pure function of the program, the launch and the
latency table, so one run per point replaces the page's repeated runs; the GPU
time of each run is reported beside it (the simulator's own speed).
"""
import json
import sys
import time

import numpy as np

from . import ks

ROOT = __import__("os").path.dirname(__import__("os").path.dirname(__import__("os").path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
from workloads import probes as P  # noqa: E402  (inputs only)


def run(w, latency=None, device="cuda:0", timed=False, reps=3):
    """Simulate one probe launch; returns (counters, ms per launch or None)."""
    import torch
    s = ks.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=w.trace_cap, latency=latency, device=device)
    try:
        s.load_gmem(w.gmem)
        s.run(w.params_bytes)
        ms = None
        if timed:
            stream = torch.cuda.current_stream(s.device)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                s.run(w.params_bytes)
            b.record(stream)
            b.synchronize()
            ms = a.elapsed_time(b) / reps
        c = s.read_counters()
        return c, ms
    finally:
        s.close()


def warp0_cycles(op, n_acc, iters, latency=None, per_iter=32, device="cuda:0"):
    c, _ = run(P.chain_probe(op, n_acc, iters, per_iter), latency=latency, device=device)
    return int(c["cycles"][0]), int(c["warp_instrs"][0])


def fit_line(x, y):
    """Least-squares y = slope * x + intercept, with R^2."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    A = np.stack([x, np.ones_like(x)], axis=1)
    (slope, intercept), *_ = np.linalg.lstsq(A, y, rcond=None)
    ss_res = float(np.sum((y - (slope * x + intercept)) ** 2))
    ss_tot = float(np.sum((y - y.mean()) ** 2))
    r2 = 1.0 if ss_tot == 0 else 1.0 - ss_res / ss_tot
    return float(slope), float(intercept), r2


def per_iteration_cycles(op, n_acc, latency=None, iters=(64, 128), device="cuda:0"):
    """Simulated cycles one more loop iteration costs (two iteration counts)."""
    (t0, _), (t1, _) = (warp0_cycles(op, n_acc, i, latency, device=device) for i in iters)
    return (t1 - t0) / (iters[1] - iters[0])


def count_sweep(op="fma.f32", n_acc=1, iters=P.COUNT_SWEEP_ITERS, per_iter=32, latency=None, device="cuda:0"):
    """Section 13: T(N) for N = iters * per_iter target instructions, fitted to L * N + C."""
    N, T = [], []
    for it in iters:
        t, _ = warp0_cycles(op, n_acc, it, latency, per_iter, device)
        N.append(it * per_iter)
        T.append(t)
    slope, intercept, r2 = fit_line(N, T)
    return {"op": op, "n_acc": n_acc, "N": N, "cycles": T, "slope": slope, "intercept": intercept, "r2": r2}


def accumulator_sweep(op="fma.f32", accs=P.ACC_SWEEP, per_iter=32, latency=None, device="cuda:0"):
    """Section 14: cycles per target instruction against the number of accumulators."""
    rows = []
    for k in accs:
        cyc = per_iteration_cycles(op, k, latency, device=device)
        prog = ks.ks_load_program(P.chain_probe_ptx(op, k, 64, per_iter))
        try:
            slots = ks.ks_program_info(prog)["reg_slots"]
        finally:
            ks.ks_program_free(prog)
        rows.append({"accumulators": k, "register_slots": slots, "cycles_per_iteration": cyc,
                     "cycles_per_instruction": cyc / per_iter, "spill_loads": 0, "spill_stores": 0})
    return rows


def control_suite(ops=P.CONTROL_OPS, n_acc=1, latency=None, device="cuda:0"):
    """Section 12: per-iteration cycles of the empty loop and of dependent chains of
    several instruction kinds; corrected = probe - empty loop."""
    empty = per_iteration_cycles("none", 1, latency, device=device)
    rows = []
    for op in ops:
        cyc = empty if op == "none" else per_iteration_cycles(op, n_acc, latency, device=device)
        rows.append({"op": op, "n_acc": n_acc, "cycles_per_iteration": cyc,
                     "corrected_cycles_per_iteration": cyc - empty})
    return rows


def warp_sweep(configs=P.WARP_SWEEP, op="fma.f32", n_acc=1, iters=512, latency=None, device="cuda:0"):
    """Section 15: the probe on more threads and warps.  Warps have independent
    scoreboards in this model, so cycles per instruction stay fixed and the
    launch's instructions per cycle grow with the warp count."""
    rows = []
    for grid, block in configs:
        w = P.chain_probe(op, n_acc, iters, grid=grid, block=block)
        c, ms = run(w, latency=latency, device=device, timed=True)
        wi = c["warp_instrs"].astype(np.int64)
        cyc = c["cycles"].astype(np.int64)
        ti = int(c["thread_instrs"].astype(np.int64).sum())
        rows.append({"blocks": grid, "threads": block, "warps": int(len(c)), "warp_instructions": int(wi.sum()),
                     "thread_instructions": ti, "max_cycles": int(cyc.max()),
                     "cycles_per_instruction": float(cyc.max()) / float(wi.max()),
                     "instructions_per_cycle": float(wi.sum()) / float(cyc.max()),
                     "gpu_ms": ms, "thread_instr_per_s": ti / (ms / 1e3) if ms else None})
    return rows


def report(device="cuda:0"):
    """All four experiments with the default latency table."""
    return {"count_sweep": [count_sweep("fma.f32", 1, device=device), count_sweep("fma.f32", 8, device=device)],
            "accumulator_sweep": accumulator_sweep(device=device),
            "controls": control_suite(device=device),
            "warp_sweep": warp_sweep(device=device)}


def main(argv=None):
    t0 = time.perf_counter()
    r = report()
    r["wall_s"] = time.perf_counter() - t0
    print(json.dumps(r, indent=1))


if __name__ == "__main__":
    main()
