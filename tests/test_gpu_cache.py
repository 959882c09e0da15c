"""GPU: the cache-latency model against the CPU oracle, bit for bit.

The model's kernels (suffix "_cache") run every workload kind with per-warp
direct-mapped L1 and L2 caches; memory, counters, trace slots and the whole
per-warp cache state (outcome counts and every tag) must equal the oracle's, and
the simulated memory must equal that of the run without the model.
"""
import numpy as np
import pytest

from workloads import configs as W
from workloads import probes as PR
from workloads import small as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from analysis_ptxsimulator_amd import ks
    ks.lib()
    return ks


def _say(msg):
    print("[gpu] " + msg, flush=True)


def cache_parity(K, O, w, cap=None, **kw):
    cap = w.trace_cap if cap is None else cap
    _say("%s grid=%s block=%s cap=%d cache" % (w.name, w.grid, w.block, cap))
    s = K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=cap, cache_model=K.KS_CACHE_WARP, **kw)
    try:
        assert s.kernel_name().endswith("_cache")
        s.load_gmem(w.gmem)
        s.run(w.params_bytes)
        gg, cg, tg = s.read_gmem(), s.read_counters(), s.read_trace()
        hg, l1g, l2g = s.read_cache()
    finally:
        s.close()
    go = w.gmem.copy()
    cache = np.zeros(w.n_warps * O.CACHE_WARP_BYTES, np.uint8)
    okw = {k: v for k, v in kw.items() if k in ("latency", "max_warp_instrs")}
    co, to, _ = O.run(w.ptx, w.grid, w.block, w.params_bytes, go, trace_cap=cap, cache=cache, **okw)
    ho, l1o, l2o = O.cache_state(cache, w.n_warps)
    assert np.array_equal(gg, go)
    for f in co.dtype.names:
        assert np.array_equal(cg[f], co[f]), f
    hgt, rg = K.trace_slots(tg, cap)
    hot, ro = O.trace_slots(to, cap)
    assert np.array_equal(hgt, hot)
    for i in range(len(hot)):  # record bytes past records_written are unspecified
        n = int(hot["records_written"][i])
        assert np.array_equal(rg[i, :n], ro[i, :n]), i
    assert np.array_equal(hg[["l1_hits", "l2_hits", "misses"]], ho[["l1_hits", "l2_hits", "misses"]])
    assert np.array_equal(l1g, l1o) and np.array_equal(l2g, l2o)
    return cg, hg


@pytest.mark.parametrize("case", ["same_line", "l1_conflict", "both_conflict", "lanes"])
def test_chase_probes(K, oracle_mod, case):
    if case == "same_line":
        w = PR.chase_probe([0, 4, 8, 12], 9, block=64, grid=2)
    elif case == "l1_conflict":
        w = PR.chase_probe([k * 1024 * 128 for k in range(5)], 15)
    elif case == "both_conflict":
        w = PR.chase_probe([k * 49152 * 128 for k in range(3)], 6)
    else:
        w = PR.chase_probe([0, 4, 8, 1 << 20, (1 << 20) + 4], 6, starts=[1 << 30, 4] + [1 << 20] * 30, block=96)
    c, h = cache_parity(K, oracle_mod, w)
    assert int(h["l1_hits"].sum() + h["l2_hits"].sum() + h["misses"].sum()) > 0


def test_vector_add(K, oracle_mod):
    cache_parity(K, oracle_mod, W.vector_add())


@pytest.mark.parametrize("s", [1, 8, 33])
def test_strided(K, oracle_mod, s):
    cache_parity(K, oracle_mod, W.strided_gather(s, n=8192))


def test_ffma(K, oracle_mod):
    cache_parity(K, oracle_mod, W.ffma_probe(8, iters=6, grid=4, block=256, trace_cap=256))


@pytest.mark.parametrize("s", [1, 32])
def test_bank(K, oracle_mod, s):
    cache_parity(K, oracle_mod, W.bank_probe(s, iters=4, grid=2, block=1024, trace_cap=64))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_stress(K, oracle_mod, seed):
    w = W.random_stress(prog_seed=seed, grid=8, block=256, gmem_bytes=1 << 24, trace_cap=1024)
    c, h = cache_parity(K, oracle_mod, w)
    assert int(h["l1_hits"].sum()) > 0 and int(h["misses"].sum()) > 0


@pytest.mark.parametrize("block", [768, 1024])
def test_random_stress_large_blocks(K, oracle_mod, block):
    """The 72-slot cache kernel (128 VGPRs, four waves per SIMD) on the largest blocks."""
    cache_parity(K, oracle_mod, W.random_stress(prog_seed=1, grid=3, block=block, gmem_bytes=1 << 24, trace_cap=300))


@pytest.mark.parametrize("seed", range(4))
def test_control_flow_shapes(K, oracle_mod, seed):
    ptx = S.random_cfg_ptx(seed, loops=seed % 2 == 1)
    n = 256
    rng = np.random.default_rng(200 + seed)
    g = np.zeros(8 * n + 4096, np.uint8)
    g[:4 * n] = rng.integers(0, 1 << 32, size=n, dtype=np.uint32).view(np.uint8)
    params = [("param_in", "u64", 0), ("param_out", "u64", 4 * n)]
    w = W.Workload(name="cfg%d" % seed, ptx=ptx, grid=(2, 1, 1), block=(128, 1, 1), params=params, gmem=g,
                   trace_cap=512)
    cache_parity(K, oracle_mod, w, max_warp_instrs=4000)


def test_faulting_lanes_and_budget(K, oracle_mod):
    data = 1 << 16
    gaddr = np.array([data + 64, 2, 30, 0] + [0] * 28, np.uint64)
    guard = np.array([1, 1, 1, 1] + [0] * 28, np.uint32)
    cache_parity(K, oracle_mod, S.addr_probe(gaddr, np.zeros(32, np.uint32), guard, data, block=32))
    cache_parity(K, oracle_mod, W.random_stress(prog_seed=0, grid=2, block=256, gmem_bytes=1 << 22, trace_cap=64),
                 max_warp_instrs=100)


def test_rerun_starts_cold(K, oracle_mod):
    """A second run sees empty caches again (ks_run clears the run's state)."""
    w = PR.chase_probe([0, 4, 8], 4)
    s = K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=8, cache_model=K.KS_CACHE_WARP)
    try:
        s.load_gmem(w.gmem)
        s.run(w.params_bytes)
        c1, h1 = s.read_counters(), s.read_cache()[0]
        s.run(w.params_bytes)
        c2, h2 = s.read_counters(), s.read_cache()[0]
    finally:
        s.close()
    assert np.array_equal(c1, c2) and np.array_equal(h1, h2)


def test_random_stress_full_size_sampled(K, oracle_mod):
    """The full 65536 x 256 random-stress launch with the cache model (105 GB of
    per-warp cache state); the oracle simulates sampled blocks, whose warps'
    counters, trace slots and cache state must match."""
    w = W.random_stress(prog_seed=0)
    blocks = [0, 1, 32767, 65535] + [int(x) for x in np.random.default_rng(7).integers(0, 65536, 4)]
    cap = w.trace_cap
    _say("%s full grid=%s cache, sampled blocks %s" % (w.name, w.grid, blocks))
    s = K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=cap, cache_model=K.KS_CACHE_WARP)
    wpb = w.warps_per_block
    try:
        s.load_gmem(w.gmem)
        s.run(w.params_bytes)
        cg = s.read_counters()
        got = []
        for b in blocks:
            hg, l1g, l2g = s.read_cache(b * wpb, wpb)
            tg = s.read_trace(b * wpb, wpb)
            got.append((hg, l1g, l2g, tg))
    finally:
        s.close()
    go = w.gmem.copy()
    cache = np.zeros(len(blocks) * wpb * oracle_mod.CACHE_WARP_BYTES, np.uint8)
    co, to, _ = oracle_mod.run(w.ptx, w.grid, w.block, w.params_bytes, go, trace_cap=cap, blocks=blocks, cache=cache)
    ho, l1o, l2o = oracle_mod.cache_state(cache, len(blocks) * wpb)
    slot = 16 + 8 * cap
    for i, b in enumerate(blocks):
        sl = slice(i * wpb, (i + 1) * wpb)
        for f in co.dtype.names:
            assert np.array_equal(cg[f][b * wpb:(b + 1) * wpb], co[f][sl]), (b, f)
        hg, l1g, l2g, tg = got[i]
        assert np.array_equal(hg[["l1_hits", "l2_hits", "misses"]], ho[sl][["l1_hits", "l2_hits", "misses"]]), b
        assert np.array_equal(l1g, l1o[sl]) and np.array_equal(l2g, l2o[sl]), b
        hgt, rg = K.trace_slots(tg, cap)
        hot, ro = oracle_mod.trace_slots(to.reshape(-1, slot)[sl].reshape(-1), cap)
        assert np.array_equal(hgt, hot), b
        for k in range(wpb):
            n = int(hot["records_written"][k])
            assert np.array_equal(rg[k, :n], ro[k, :n]), (b, k)
