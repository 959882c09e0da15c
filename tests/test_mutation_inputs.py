"""CPU: the mutant generator (workloads/mutate.py) is deterministic, keeps most
mutants inside the grammar both parsers accept, and the oracle finishes every
mutant under an issue budget (loops made by retargeted branches end there)."""
import random

import pytest

from workloads import mutate as M


@pytest.fixture(scope="module")
def ks():
    from analysis_ptxsimulator_amd import build, ks as K
    build.build(force=False)
    return K


def test_mutants_are_seeded():
    a = [M.mutate(random.Random(7), t) for t in M.base_programs()]
    b = [M.mutate(random.Random(7), t) for t in M.base_programs()]
    assert a == b
    assert sum(x != y for x, y in zip(a, M.base_programs())) > len(a) // 2


def test_mutants_parse_and_finish(ks, oracle_mod):
    rnd = random.Random(11)
    bases = M.base_programs()
    loaded = ran = budget_stops = 0
    for _ in range(300):
        text = M.mutate(rnd, rnd.choice(bases))
        try:
            params = oracle_mod.params(text)
            p = ks.ks_load_program(text)
            ks.ks_program_free(p)
        except (oracle_mod.OracleError, ks.KsError):
            continue
        loaded += 1
        w = M.workload(rnd, text, params)
        c, _, _ = oracle_mod.run(text, w.grid, w.block, w.params_bytes, w.gmem.copy(), max_warp_instrs=700)
        assert (c["warp_instrs"] <= 700).all()
        assert (c["status"] & (oracle_mod.ST_FINISHED | oracle_mod.ST_BUDGET)).all()
        budget_stops += int((c["status"] & oracle_mod.ST_BUDGET).any())
        ran += 1
    assert loaded > 270 and ran == loaded
    assert budget_stops > 0  # some mutants loop until the budget
