"""GPU: a seeded randomised sweep of run shapes against the CPU oracle, bit for bit.

Each case draws a workload shape and the run's options independently:
- random_stress programs of 300-2000 instructions (every instruction class of the
  subset, divergent forward branches, barriers at converged points) on 1-69
  blocks of 32-1024 threads, or small random control-flow programs (guarded
  branches and predicated ret over per-lane data) on one or more blocks;
- trace caps around the 32-record chunk boundaries and past the program length,
  issue budgets that stop warps early, basic or extended records (extended runs
  of more than 32 blocks go out in several launches), and the cache-latency
  model.
Memory, every counter field, every trace header, every written record and (with
the cache model) every tag of every warp must equal the oracle's.
"""
import numpy as np
import pytest

from workloads import configs as W
from workloads import small as S

pytestmark = pytest.mark.gpu

N_CASES = 300


@pytest.fixture(scope="module")
def K():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from analysis_ptxsimulator_amd import ks
    ks.lib()
    return ks


def _case(rng):
    """One workload and run options, drawn from rng."""
    fmt = int(rng.choice([0, 1]))
    cache = (not fmt) and bool(rng.random() < 0.4)
    budget = int(rng.choice([0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 40, 777]))
    if rng.random() < 0.75:
        seed = int(rng.integers(0, 5000))
        # extended records on blocks of up to 256 threads here (larger ones: test_gpu_ext_trace)
        block = int(rng.choice([32, 64, 96, 160, 256] + ([] if fmt else [512, 768, 1024])))
        grid = int(rng.integers(1, 70))
        cap = int(rng.choice([0, 1, 17, 31, 32, 33, 64, 300, 2048]))
        w = W.random_stress(prog_seed=seed, grid=grid, block=block, gmem_bytes=1 << 23, trace_cap=cap,
                            n_instr=int(rng.integers(300, 2000)))
        desc = "random_stress seed=%d grid=%d block=%d n_instr=%d" % (seed, grid, block, w.meta["n_instr"])
    else:
        seed = int(rng.integers(0, 100000))
        n = 256
        data = rng.choice([0, 1, 500, 1500, 2500, 2999], size=n).astype(np.uint32)
        g = np.zeros(8 * n + 4096, np.uint8)
        g[:4 * n] = data.view(np.uint8)
        block = int(rng.choice([32, 64, 128, 256]))
        cap = int(rng.choice([0, 5, 32, 128]))
        w = W.Workload(name="cfg%d" % seed, ptx=S.random_cfg_ptx(seed, n_instr=int(rng.integers(8, 60))),
                       grid=(n // block, 1, 1), block=(block, 1, 1),
                       params=[("param_in", "u64", 0), ("param_out", "u64", 4 * n)], gmem=g, trace_cap=cap)
        desc = "random_cfg seed=%d block=%d" % (seed, block)
    return w, cap, fmt, cache, budget, desc


def _compare(K, O, w, cap, fmt, cache, budget, latency=None):
    kw = dict(trace_cap=cap, trace_format=fmt, max_warp_instrs=budget, latency=latency)
    if cache:
        kw["cache_model"] = K.KS_CACHE_WARP
    s = K.Session(w.ptx, w.grid, w.block, w.gmem.size, **kw)
    try:
        s.load_gmem(w.gmem)
        s.trace.zero_()
        s.run(w.params_bytes)
        gg, cg, tg = s.read_gmem(), s.read_counters(), s.read_trace()
        cs = s.read_cache() if cache else None
    finally:
        s.close()
    go = w.gmem.copy()
    ofmt = O.TRACE_EXTENDED if fmt else O.TRACE_BASIC
    okw = dict(trace_cap=cap, max_warp_instrs=budget, trace_format=ofmt, latency=latency)
    cbuf = None
    if cache:
        cbuf = np.zeros(w.n_warps * O.CACHE_WARP_BYTES, np.uint8)
        okw["cache"] = cbuf
    co, to, _ = O.run(w.ptx, w.grid, w.block, w.params_bytes, go, **okw)
    bad = []
    if not np.array_equal(gg, go):
        bad.append("memory")
    bad += ["counter " + f for f in co.dtype.names if not np.array_equal(cg[f], co[f])]
    hg, rg = K.trace_slots(tg, cap, fmt)
    ho, ro = O.trace_slots(to, cap, ofmt)
    if not np.array_equal(hg, ho):
        bad.append("trace headers")
    for i in range(len(ho)):  # record bytes past records_written are unspecified
        n = int(ho["records_written"][i])
        if not np.array_equal(rg[i, :n], ro[i, :n]):
            bad.append("records of warp %d" % i)
            break
    if cache:
        ho2, l1o, l2o = O.cache_state(cbuf, w.n_warps)
        hgc, l1g, l2g = cs
        if not (np.array_equal(hgc[["l1_hits", "l2_hits", "misses"]], ho2[["l1_hits", "l2_hits", "misses"]])
                and np.array_equal(l1g, l1o) and np.array_equal(l2g, l2o)):
            bad.append("cache state")
    return bad


def test_random_sweep(K, oracle_mod):
    rng = np.random.default_rng(20261202)
    failures = []
    for t in range(N_CASES):
        w, cap, fmt, cache, budget, desc = _case(rng)
        line = "case %d: %s cap=%d %s%s budget=%d" % (t, desc, cap, "extended" if fmt else "basic",
                                                      " cache" if cache else "", budget)
        print("[gpu] " + line, flush=True)
        bad = _compare(K, oracle_mod, w, cap, fmt, cache, budget)
        if bad:
            failures.append("%s: %s" % (line, ", ".join(bad)))
    assert not failures, "\n".join(failures)
