"""GPU: seeded mutants of valid programs against the CPU oracle, bit for bit.

Each mutant changes registers, guards, branch targets (loops included), inserts
barriers (also in divergent code), changes comparisons and immediates, or
duplicates or deletes lines (workloads/mutate.py).  Mutants the oracle's race
checker flags are skipped, since their results may depend on the order blocks
and warps run in; every other one runs under an issue budget with a trace cap,
record format and cache model drawn per case, on 1-D launches of whole warps in
the first test and on 2-D and 3-D launches of ragged warps with caller-set
latency tables (0 and 65535 included) in the second.  Memory, every counter
field, every trace header and written record, and the cache tags must equal the
oracle's.
"""
import random

import numpy as np
import pytest

from workloads import mutate as M

pytestmark = pytest.mark.gpu

N_CASES = 3000


@pytest.fixture(scope="module")
def K():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from analysis_ptxsimulator_amd import ks
    ks.lib()
    return ks


@pytest.mark.parametrize("shapes", ["whole_warps", "ragged_latency"])
def test_mutated_programs(K, oracle_mod, shapes):
    from .test_gpu_sweep import _compare
    rnd = random.Random(20261202 if shapes == "whole_warps" else 20261203)
    bases = M.base_programs()
    failures = []
    compared = 0
    for t in range(N_CASES):
        text = M.mutate(rnd, rnd.choice(bases))
        try:
            params = oracle_mod.params(text)
            p = K.ks_load_program(text)
            K.ks_program_free(p)
        except (oracle_mod.OracleError, K.KsError):
            continue
        w = M.workload(rnd, text, params)
        lat = None
        budget = rnd.choice([3000, 700])
        if shapes == "ragged_latency":
            w.grid, w.block = M.launch_shape(rnd)
            if rnd.random() < 0.6:
                lat = M.latency_table(rnd, oracle_mod.NLAT)
                budget = rnd.choice([700, 3000, 40000])
        _, _, rc = oracle_mod.run(text, w.grid, w.block, w.params_bytes, w.gmem.copy(), max_warp_instrs=budget,
                                  check_races=True, latency=lat)
        if rc == oracle_mod.E_RACE:
            continue
        cap = rnd.choice([0, 33, 512])
        fmt = rnd.choice([0, 1])
        cache = (not fmt) and rnd.random() < 0.3
        w.trace_cap = cap
        line = "mutant %d: grid %s block %s cap %d %s%s budget %d latency %s" % (
            t, w.grid, w.block, cap, "extended" if fmt else "basic", " cache" if cache else "", budget, lat)
        print("[gpu] " + line, flush=True)
        bad = _compare(K, oracle_mod, w, cap, fmt, cache, budget, lat)
        compared += 1
        if bad:
            failures.append("%s: %s\n%s" % (line, ", ".join(bad), text))
    assert compared > N_CASES // 2
    assert not failures, "\n\n".join(failures[:3])
