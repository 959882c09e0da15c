"""GPU: extended 16-byte trace records against the CPU oracle, bit for bit.

The extended format runs the interpreter variants that write {issue cycle, pc,
kind, active mask, payload} per issued instruction; memory, counters, headers
and every written record must equal the oracle's, and the basic-format run of
the same inputs must give the same memory and counters.
"""
import numpy as np
import pytest

from workloads import configs as W
from workloads import probes as PR
from workloads import small as S
from workloads.configs import pack_params

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


def gpu_run(K, w, fmt, cap, **kw):
    _say("%s grid=%s block=%s cap=%d format=%d" % (w.name, w.grid, w.block, cap, fmt))
    s = K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=cap, trace_format=fmt, **kw)
    try:
        s.load_gmem(w.gmem)
        s.run(w.params_bytes)
        name = s.kernel_name()
        return s.read_gmem(), s.read_counters(), s.read_trace(), name
    finally:
        s.close()


def ext_parity(K, O, w, cap=None, **kw):
    cap = w.trace_cap if cap is None else cap
    gg, cg, tg, name = gpu_run(K, w, K.KS_TRACE_EXTENDED, cap, **kw)
    assert name.endswith("_ext")
    go = w.gmem.copy()
    okw = {k: v for k, v in kw.items() if k in ("latency", "max_warp_instrs")}
    co, to, _ = O.run(w.ptx, w.grid, w.block, w.params_bytes, go, trace_cap=cap, trace_format=O.TRACE_EXTENDED, **okw)
    assert np.array_equal(gg, go)
    for f in co.dtype.names:
        assert np.array_equal(cg[f], co[f]), f
    hg, rg = K.trace_slots(tg, cap, K.KS_TRACE_EXTENDED)
    ho, ro = O.trace_slots(to, cap, O.TRACE_EXTENDED)
    assert np.array_equal(hg, ho)
    for i in range(len(ho)):
        n = int(ho["records_written"][i])
        assert np.array_equal(rg[i, :n], ro[i, :n]), i
    # the basic format of the same run: same memory and counters
    gb, cb, _, _ = gpu_run(K, w, K.KS_TRACE_BASIC, cap, **kw)
    assert np.array_equal(gb, gg) and np.array_equal(cb, cg)


def test_vector_add(K, oracle_mod):
    ext_parity(K, oracle_mod, W.vector_add())


@pytest.mark.parametrize("s", [1, 3, 33])
def test_strided(K, oracle_mod, s):
    ext_parity(K, oracle_mod, W.strided_gather(s, n=8192))


@pytest.mark.parametrize("n_acc", [1, 8])
def test_ffma(K, oracle_mod, n_acc):
    ext_parity(K, oracle_mod, W.ffma_probe(n_acc, iters=6, grid=4, block=256, trace_cap=256))


@pytest.mark.parametrize("s", [1, 7, 32])
def test_bank(K, oracle_mod, s):
    ext_parity(K, oracle_mod, W.bank_probe(s, iters=4, grid=2, block=256, trace_cap=64))


@pytest.mark.parametrize("s", [1, 7, 32])
def test_bank_block_1024(K, oracle_mod, s):
    """Four waves per SIMD: blocks of 1024 threads."""
    ext_parity(K, oracle_mod, W.bank_probe(s, iters=4, grid=2, block=1024, trace_cap=64))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_stress(K, oracle_mod, seed):
    ext_parity(K, oracle_mod, W.random_stress(prog_seed=seed, grid=8, block=256, gmem_bytes=1 << 24,
                                              trace_cap=1024))


def test_random_stress_cap_overflow(K, oracle_mod):
    """Records past the cap dropped and counted; blocks above the 64-slot extended
    variant's largest are refused."""
    ext_parity(K, oracle_mod, W.random_stress(prog_seed=2, grid=3, block=256, gmem_bytes=1 << 24, trace_cap=300))
    w = W.random_stress(prog_seed=2, grid=1, block=1024, gmem_bytes=1 << 22, trace_cap=8)
    with pytest.raises(K.KsError, match="768"):
        K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=8, trace_format=K.KS_TRACE_EXTENDED)


def test_long_program(K, oracle_mod):
    """A 32000-instruction random program: pcs above 2^14 in the 16-bit record
    field, and a 1024-record cap against about 31000 issues per warp."""
    ext_parity(K, oracle_mod, W.random_stress(prog_seed=7, grid=2, block=64, gmem_bytes=1 << 22, trace_cap=1024,
                                              n_instr=32000))


def test_random_stress_block_768(K, oracle_mod):
    """The 64-slot extended kernel's largest block: three waves per SIMD."""
    ext_parity(K, oracle_mod, W.random_stress(prog_seed=2, grid=3, block=768, gmem_bytes=1 << 24, trace_cap=300))


def test_budget_stop_at_a_barrier(K, oracle_mod):
    """Warps whose budget ends exactly at a bar.sync report cycles = that issue + 1."""
    w = W.random_stress(prog_seed=989, grid=30, block=64, gmem_bytes=1 << 22, trace_cap=33, n_instr=1106)
    ext_parity(K, oracle_mod, w, max_warp_instrs=777)


def test_random_stress_chunked_launches(K, oracle_mod):
    """A grid above KS_EXT_MAX_BLOCKS runs as consecutive launches of that many
    blocks (here 32 + 32 + 16): every byte equal to the oracle's."""
    ext_parity(K, oracle_mod, W.random_stress(prog_seed=1, grid=80, block=256, gmem_bytes=1 << 24, trace_cap=512))


def test_random_stress_full_grid_extended(K, oracle_mod):
    """The whole 65536 x 256 grid with extended records (2048 launches of 32 blocks;
    the 17.2 GB of slots reach far past 4 GiB): memory and every counter record
    equal the basic-format run of the same inputs, every header agrees with its
    warp's issue count, and the records of sampled blocks (the first, the last
    and blocks whose slots lie past 4 GiB) equal the oracle's."""
    w = W.random_stress(prog_seed=0)
    cap = w.trace_cap
    _say("full grid, basic format")
    sb = K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=cap)
    try:
        sb.load_gmem(w.gmem)
        sb.run(w.params_bytes)
        gb, cb = sb.read_gmem(), sb.read_counters()
    finally:
        sb.close()
    _say("full grid, extended format")
    se = K.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=cap, trace_format=K.KS_TRACE_EXTENDED)
    try:
        se.load_gmem(w.gmem)
        se.run(w.params_bytes)
        assert se.kernel_name() == "ks_interp_v64_ext"
        assert np.array_equal(se.read_gmem(), gb)
        ce = se.read_counters()
        assert np.array_equal(ce, cb)
        wpb = w.warps_per_block
        slot = 16 + 16 * cap
        hdr = np.empty(len(ce), dtype=K.TRACE_HEADER_DTYPE)
        step = 8192  # warps per read: headers only are checked over the whole grid
        for w0 in range(0, len(ce), step):
            h, _ = K.trace_slots(se.read_trace(w0, min(step, len(ce) - w0)), cap, K.KS_TRACE_EXTENDED)
            hdr[w0:w0 + len(h)] = h
        wi = ce["warp_instrs"].astype(np.int64)
        assert np.array_equal(hdr["records_written"], np.minimum(wi, cap))
        assert np.array_equal(hdr["records_dropped"].astype(np.int64), wi - np.minimum(wi, cap))
        assert (hdr["version"] == 2).all()
        blocks = [0, 16383, 16384, 40000, 65535]  # slots of block 16384 on start past 4 GiB
        assert 16384 * wpb * slot >= 1 << 32
        go = w.gmem.copy()
        co, to, _ = oracle_mod.run(w.ptx, w.grid, w.block, w.params_bytes, go, trace_cap=cap, blocks=blocks,
                                   trace_format=oracle_mod.TRACE_EXTENDED)
        ho, ro = oracle_mod.trace_slots(to, cap, oracle_mod.TRACE_EXTENDED)
        for j, b in enumerate(blocks):
            hg, rg = K.trace_slots(se.read_trace(b * wpb, wpb), cap, K.KS_TRACE_EXTENDED)
            assert np.array_equal(hg, ho[j * wpb:(j + 1) * wpb]), b
            for i in range(wpb):
                n = int(hg["records_written"][i])
                assert np.array_equal(rg[i, :n], ro[j * wpb + i, :n]), (b, i)
            assert np.array_equal(ce[b * wpb:(b + 1) * wpb], co[j * wpb:(j + 1) * wpb]), b
    finally:
        se.close()


@pytest.mark.parametrize("op", ["fma.f32", "mad.s32", "none"])
def test_probe_chains(K, oracle_mod, op):
    ext_parity(K, oracle_mod, PR.chain_probe(op, 3, 5, grid=3, block=96, trace_cap=256))


@pytest.mark.parametrize("seed", range(6))
def test_control_flow_shapes(K, oracle_mod, seed):
    ptx = S.random_cfg_ptx(seed, loops=seed % 2 == 1)
    n = 256
    rng = np.random.default_rng(100 + seed)
    g = np.zeros(8 * n + 4096, np.uint8)
    g[:4 * n] = rng.integers(0, 1 << 32, size=n, dtype=np.uint32).view(np.uint8)
    params = [("param_in", "u64", 0), ("param_out", "u64", 4 * n)]
    w = W.Workload(name="cfg%d" % seed, ptx=ptx, grid=(2, 1, 1), block=(128, 1, 1), params=params, gmem=g,
                   trace_cap=512)
    ext_parity(K, oracle_mod, w, max_warp_instrs=4000)


def test_faulting_and_misaligned_lanes(K, oracle_mod):
    data = 1 << 16
    gaddr = np.array([0, 2, 30, data + 64] + [0] * 28, np.uint64)
    guard = np.array([1, 1, 1, 1] + [0] * 28, np.uint32)
    w = S.addr_probe(gaddr, np.zeros(32, np.uint32), guard, data, block=32)
    ext_parity(K, oracle_mod, w)


def test_budget(K, oracle_mod):
    ext_parity(K, oracle_mod, W.random_stress(prog_seed=0, grid=2, block=256, gmem_bytes=1 << 22, trace_cap=64),
               max_warp_instrs=100)


@pytest.mark.parametrize("case", ["bank_8", "strided_33", "random_1"])
def test_host_analysis_on_gpu_records(K, oracle_mod, case):
    """Hints and the trace-event export computed from the GPU's extended records
    equal those computed from the oracle's."""
    from analysis_ptxsimulator_amd import analysis as A
    kind, arg = case.split("_")
    if kind == "bank":
        w = W.bank_probe(int(arg), iters=3, grid=2, block=256, trace_cap=64)
    elif kind == "strided":
        w = W.strided_gather(int(arg), n=4096)
    else:
        w = W.random_stress(prog_seed=int(arg), grid=2, block=256, gmem_bytes=1 << 22, trace_cap=2048)
    _, _, tg, _ = gpu_run(K, w, K.KS_TRACE_EXTENDED, w.trace_cap)
    go = w.gmem.copy()
    _, to, _ = oracle_mod.run(w.ptx, w.grid, w.block, w.params_bytes, go, trace_cap=w.trace_cap,
                              trace_format=oracle_mod.TRACE_EXTENDED)
    info = A.ProgramInfo(w.ptx)
    occ = A.program_occupancy(w.ptx, w.threads_per_block)
    hg, rg = K.trace_slots(tg, w.trace_cap, K.KS_TRACE_EXTENDED)
    ho, ro = oracle_mod.trace_slots(to, w.trace_cap, oracle_mod.TRACE_EXTENDED)
    assert A.hints(hg, rg, info, occ, w.warps_per_block) == A.hints(ho, ro, info, occ, w.warps_per_block)
    assert A.chrome_trace(hg, rg, info, w.warps_per_block) == A.chrome_trace(ho, ro, info, w.warps_per_block)


def test_analysis_command_on_a_ptx_file(K, oracle_mod, tmp_path, capsys):
    """The analysis command on a user's PTX file: vector_add with its launch shape,
    parameters and memory image given on the command line reports the same hints
    as the built-in vector_add workload, and writes its trace-event file."""
    import json
    from analysis_ptxsimulator_amd import analysis as A
    w = W.vector_add()
    ptx = tmp_path / "vadd.ptx"
    ptx.write_text(w.ptx)
    img = tmp_path / "mem.bin"
    w.gmem.tofile(str(img))
    out = tmp_path / "trace.json"
    A.main(["--ptx", str(ptx), "--grid", "4", "--block", "256", "--gmem", str(img), "--trace-cap", "32",
            "--param", "param_a=0", "--param", "param_b=4096", "--param", "param_c=0x2000", "--param", "param_n=1000",
            "--out", str(out), "--dump-gmem", str(tmp_path / "after.bin")])
    got = json.loads(capsys.readouterr().out)
    c = np.fromfile(str(tmp_path / "after.bin"), np.uint8)[0x2000:0x2000 + 4000].view(np.float32)
    a, b = w.gmem[:4000].view(np.float32), w.gmem[4096:8096].view(np.float32)
    assert np.array_equal(c, a + b)  # the memory after the run: c = a + b
    assert got["counters"]["thread_instrs"] == 19264 and got["counters"]["max_cycles"] == 239
    A.main(["--workload", "vector_add"])
    ref = json.loads(capsys.readouterr().out)
    assert got["workload"] == "vadd.ptx" and got["kernel"] == ref["kernel"]
    assert got["occupancy"] == ref["occupancy"] and got["hints"] == ref["hints"]
    assert got["n_event_hints"] == ref["n_event_hints"]
    events = json.load(open(out))
    assert len(events["traceEvents"]) > 32
