"""Pins of the cache-latency model on the CPU oracle.

The model is the KernelScope page's (simulator part, memory analysis: cache
parameters and SimpleCache): direct-mapped L1 of 1024 and L2 of 49152 lines of
128 bytes, L1 hit 28 cycles, L2 hit 150, DRAM 400, looked up with one
representative address per warp access.  Reading: the caches are private to each
warp (so that the result does not depend on how warps interleave) and the
representative is the lowest guard lane whose access is valid.

Every pin runs the pointer-chase probe (workloads/probes.py), a chain of
dependent loads: the issue cycle of each hop is the previous hop's plus the load
latency plus the 8 cycles of mul.wide and add.s64, so the run's cycles with the
cache model minus its cycles with the fixed ld.global latency (200) are exactly
the sum over the loads of (cache latency - 200).  Chains whose lines share an L1
set, or an L1 and an L2 set, fix which level each hop reaches.
"""
import numpy as np
import pytest

from workloads import probes as PR

L1_SETS, L2_SETS, LINE = 1024, 49152, 128
L1, L2, DRAM, FIXED = 28, 150, 400, 200


def run_both(O, w, latency=None):
    g0 = w.gmem.copy()
    c0, _, _ = O.run(w.ptx, w.grid, w.block, w.params_bytes, g0, trace_cap=0, latency=latency)
    g1 = w.gmem.copy()
    cache = np.zeros(w.n_warps * O.CACHE_WARP_BYTES, np.uint8)
    c1, _, _ = O.run(w.ptx, w.grid, w.block, w.params_bytes, g1, trace_cap=0, cache=cache, latency=latency)
    assert np.array_equal(g0, g1)  # the model changes timing only
    hdr, l1, l2 = O.cache_state(cache, w.n_warps)
    return c0, c1, hdr, l1, l2


def tags_of(lines, sets):
    t = {}
    for ln in lines:
        t[ln % sets] = ln + 1
    return t


def check_tags(arr, expect):
    nz = {int(i): int(arr[i]) for i in np.nonzero(arr)[0]}
    assert nz == expect


@pytest.mark.parametrize("hops", [1, 2, 7])
def test_same_line_chain(oracle_mod, hops):
    """Every hop inside line 0: the first reaches DRAM, the rest hit the L1."""
    w = PR.chase_probe([0, 4, 8, 12, 16, 20, 24, 28], hops)
    c0, c1, hdr, l1, l2 = run_both(oracle_mod, w)
    start, out = w.meta["off_start"] // LINE, w.meta["off_out"] // LINE
    lat = [DRAM] + [DRAM] + [L1] * (hops - 1)  # start-table load, then the hops
    assert int(c1["cycles"][0]) - int(c0["cycles"][0]) == sum(x - FIXED for x in lat)
    assert (hdr["l1_hits"][0], hdr["l2_hits"][0], hdr["misses"][0]) == (hops - 1, 0, 3)  # + the store's miss
    check_tags(l1[0], tags_of([start, 0, out], L1_SETS))
    check_tags(l2[0], tags_of([start, 0, out], L2_SETS))


@pytest.mark.parametrize("m", [2, 5])
def test_l1_conflicts_hit_the_l2(oracle_mod, m):
    """Lines 1024 apart share L1 set 0 but not an L2 set: after the first pass every
    hop misses the L1 and hits the L2."""
    cycle = [k * L1_SETS * LINE for k in range(m)]
    w = PR.chase_probe(cycle, 3 * m)
    c0, c1, hdr, l1, l2 = run_both(oracle_mod, w)
    lat = [DRAM] + [DRAM] * m + [L2] * (2 * m)
    assert int(c1["cycles"][0]) - int(c0["cycles"][0]) == sum(x - FIXED for x in lat)
    assert (hdr["l1_hits"][0], hdr["l2_hits"][0], hdr["misses"][0]) == (0, 2 * m, m + 2)
    lines = [c // LINE for c in cycle]
    start, out = w.meta["off_start"] // LINE, w.meta["off_out"] // LINE
    check_tags(l2[0], tags_of([start] + lines + [out], L2_SETS))
    # L1 set 0 keeps the last chain line read: hop 3m reads cycle[(3m - 1) mod m]
    check_tags(l1[0], tags_of([start, cycle[(3 * m - 1) % m] // LINE, out], L1_SETS))


@pytest.mark.parametrize("m", [2, 3])
def test_l1_and_l2_conflicts_reach_dram(oracle_mod, m):
    """Lines 49152 apart share L1 set 0 and L2 set 0: every hop reaches DRAM."""
    cycle = [k * L2_SETS * LINE for k in range(m)]
    w = PR.chase_probe(cycle, 2 * m)
    c0, c1, hdr, _, _ = run_both(oracle_mod, w)
    lat = [DRAM] * (1 + 2 * m)
    assert int(c1["cycles"][0]) - int(c0["cycles"][0]) == sum(x - FIXED for x in lat)
    assert (hdr["l1_hits"][0], hdr["l2_hits"][0], hdr["misses"][0]) == (0, 0, 2 * m + 2)


@pytest.mark.parametrize("l1,l2,dram", [(0, 0, 0), (0, 7, 1000), (5, 0, 65535), (1, 1, 1)])
def test_level_latencies_come_from_the_table(oracle_mod, l1, l2, dram):
    """Caller-set L1, L2 and DRAM latencies, 0 included: a hop that looked up a level
    takes that level's table value.  A load issued at t makes its value ready at
    t + x and the dependent mul.wide issues no earlier than t + 1, so a load of
    latency x costs max(x, 1) cycles before the next hop; after the last load the
    independent add.s64 issues at t + 1 and the store waits for it until t + 5, so
    the last load costs max(x, 5).  With the fixed ld.global latency every load
    costs 200."""
    lat = oracle_mod.default_latency()
    lat[14], lat[15], lat[16] = l1, l2, dram

    def cost(loads):
        return sum(max(x, 1) - FIXED for x in loads[:-1]) + max(loads[-1], 5) - FIXED

    w = PR.chase_probe([0, 4, 8, 12], 4)
    c0, c1, _, _, _ = run_both(oracle_mod, w, lat)
    assert int(c1["cycles"][0]) - int(c0["cycles"][0]) == cost([dram, dram, l1, l1, l1])
    m = 2
    w = PR.chase_probe([k * L1_SETS * LINE for k in range(m)], 3 * m)
    c0, c1, _, _, _ = run_both(oracle_mod, w, lat)
    assert int(c1["cycles"][0]) - int(c0["cycles"][0]) == cost([dram] + [dram] * m + [l2] * (2 * m))


def test_representative_is_the_lowest_valid_lane(oracle_mod):
    """Only lane 0's chain reaches the caches; with lane 0's start invalid (its loads
    fault) lane 1's does."""
    a = [0, 4, 8]                                       # line 0
    b = [1 << 20, (1 << 20) + 4, (1 << 20) + 8]         # line 8192 (L1 set 0, L2 set 8192)
    w = PR.chase_probe(a + b, 4, starts=[0] + [1 << 20] * 31)
    c0, c1, hdr, l1, l2 = run_both(oracle_mod, w)
    # lane 0 reads 0 (DRAM), 4 and 8 (L1 hits), then 1 MiB: line 8192 shares L1 set 0
    # with line 0 and misses both levels; plus the start table's and the store's misses
    assert (hdr["l1_hits"][0], hdr["l2_hits"][0], hdr["misses"][0]) == (2, 0, 4)
    assert int(c1["cycles"][0]) - int(c0["cycles"][0]) == sum(x - FIXED for x in [DRAM, DRAM, L1, L1, DRAM])
    w2 = PR.chase_probe(a + b, 4, starts=[0] + [8] * 31)
    _, c2, hdr2, l1b, l2b = run_both(oracle_mod, w2)
    assert int(c2["cycles"][0]) == int(c1["cycles"][0])
    assert np.array_equal(hdr2, hdr) and np.array_equal(l1b, l1) and np.array_equal(l2b, l2)
    # lane 0 starts out of range: its loads fault (and read 0), lane 1 leads
    bad = len(w.gmem) + 4096
    w3 = PR.chase_probe(a + b, 1, starts=[bad] + [1 << 20] * 31)
    _, c3, hdr3, l13, _ = run_both(oracle_mod, w3)
    assert int(c3["fault_n"][0]) == 1
    line_b = (1 << 20) // LINE
    assert int(l13[0][line_b % L1_SETS]) == line_b + 1


def test_no_valid_lane_takes_the_table_latency(oracle_mod):
    """A load whose every guard lane faults touches no cache and takes the ld.global
    latency; the next hop (address 0, what the faulting loads read) reaches DRAM."""
    w = PR.chase_probe([0, 4], 2, starts=[1 << 30])
    c0, c1, hdr, _, _ = run_both(oracle_mod, w)
    assert int(c1["fault_n"][0]) == 32
    lat = [DRAM, FIXED, DRAM]  # start table, the faulting hop, hop 2 at address 0
    assert int(c1["cycles"][0]) - int(c0["cycles"][0]) == sum(x - FIXED for x in lat)
    assert (hdr["l1_hits"][0], hdr["l2_hits"][0], hdr["misses"][0]) == (0, 0, 3)


def test_caches_are_private_per_warp(oracle_mod):
    """Two warps (and two blocks) chasing the same chain see the same cold caches."""
    w = PR.chase_probe([0, 4, 8], 3, block=64, grid=2)
    _, c1, hdr, l1, l2 = run_both(oracle_mod, w)
    assert len(set(int(x) for x in c1["cycles"])) == 1
    assert all(np.array_equal(hdr[k], hdr[0]) for k in range(4))
    assert tuple(hdr[0])[:3] == (2, 0, 3)
    for k in range(4):  # warp k's own start-table and output lines, and the chain's line 0
        start = (w.meta["off_start"] + 128 * (k % 2)) // LINE  # rows by %tid.x
        out = (w.meta["off_out"] + 128 * (k % 2)) // LINE
        check_tags(l1[k], tags_of([start, 0, out], L1_SETS))
        check_tags(l2[k], tags_of([start, 0, out], L2_SETS))
