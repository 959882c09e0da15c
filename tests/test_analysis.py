"""Host analysis: occupancy model, hint rules and the trace-event export.

The occupancy model is pinned by the KernelScope page's worked example (sm_80,
256 threads per block: 32 registers per thread give 64 active warps, 100%; 128
registers give 25%) and by hand-computed cases for each limiter.  The hint rules
run over extended trace records of the CPU oracle, on workloads whose memory
pattern fixes the answer (bank-conflict degree gcd(s, 32), strided sectors
min(32, 4 s)); the export is checked field by field against the hand-derived
vector_add trace in tests/golden.
"""
import ctypes
import json
import math
import os

import numpy as np
import pytest

from workloads import configs as W
from workloads import small as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def A():
    from analysis_ptxsimulator_amd import analysis, build
    build.build(force=False)
    return analysis


def ext(O, w, cap=None):
    cap = w.trace_cap if cap is None else cap
    g = w.gmem.copy()
    c, t, _ = O.run(w.ptx, w.grid, w.block, w.params_bytes, g, trace_cap=cap, trace_format=O.TRACE_EXTENDED)
    return c, O.trace_slots(t, cap, O.TRACE_EXTENDED)


def test_occupancy_page_example(A):
    r = A.occupancy("sm_80", 256, 32)
    assert r["active_warps_per_sm"] == 64 and r["occupancy_percent"] == 100.0
    assert r["warps_by_registers"] == 64 and r["warps_by_block_size"] == 64
    assert r["limiting_factor"] == "registers"
    r = A.occupancy("sm_80", 256, 128)
    assert r["active_warps_per_sm"] == 16 and r["occupancy_percent"] == 25.0 and r["limiting_factor"] == "registers"


def test_occupancy_limiters_by_hand(A):
    # 33 registers: 33 * 32 = 1056 -> 1280 per warp (groups of 256); 65536 // 1280 = 51 warps
    r = A.occupancy("sm_80", 128, 33)
    assert r["warps_by_registers"] == 51 and r["active_warps_per_sm"] == 51
    # 48 KiB of shared memory per block: 167936 // 49152 = 3 blocks of 8 warps
    r = A.occupancy("sm_80", 256, 0, 48 * 1024)
    assert r["active_warps_per_sm"] == 24 and r["limiting_factor"] == "shared_memory"
    assert r["occupancy_percent"] == 37.5
    # 100 bytes of shared memory round up to 256: 65536 // 256 = 256 blocks, capped elsewhere
    r = A.occupancy("sm_75", 32, 0, 100)
    assert r["warps_by_shared_memory"] == 256 and r["active_warps_per_sm"] == 16
    assert r["limiting_factor"] == "block_size"  # 16 blocks per SM of 1 warp
    # one 1024-thread block fills a T4's 32 warps
    r = A.occupancy("sm_75", 1024, 16)
    assert r["active_warps_per_sm"] == 32 and r["occupancy_percent"] == 100.0
    r = A.occupancy("sm_86", 1024, 0)
    assert r["active_warps_per_sm"] == 32 and r["limiting_factor"] == "block_size"
    with pytest.raises(ValueError):
        A.occupancy("sm_80", 2048, 32)


def test_program_occupancy_uses_declared_registers(A):
    w = W.bank_probe(1, iters=1, grid=1, block=1024)
    r = A.program_occupancy(w.ptx, 1024)
    from analysis_ptxsimulator_amd import ks
    p = ks.ks_load_program(w.ptx)
    info = ks.ks_program_info(p)
    ks.ks_program_free(p)
    assert r == A.occupancy("sm_80", 1024, info["reg_slots"], info["shared_bytes"])


@pytest.mark.parametrize("s", [1, 2, 4, 8, 16, 32, 33])
def test_bank_conflict_hints(A, oracle_mod, s):
    w = W.bank_probe(s, iters=2, grid=1, block=256, trace_cap=64)
    _, (hdr, rec) = ext(oracle_mod, w)
    info = A.ProgramInfo(w.ptx)
    hs = A.hints(hdr, rec, info, warps_per_block=w.warps_per_block)
    d = math.gcd(s, 32)
    per_event = [h for h in hs if "warp" in h and "bank-conflict degree" in h["message"]]
    # the probe's one global load of v[lane * s] touches min(32, s) lines for 128
    # requested bytes (one line's worth): below 25% efficiency (critical) past 4 lines
    scattered = [h for h in hs if "efficiency" in h]
    assert len(scattered) == (8 if min(32, s) > 4 else 0)
    assert all(abs(h["efficiency"] - 1.0 / min(32, s)) < 1e-12 for h in scattered)
    if d == 1:
        assert per_event == []
    else:
        assert len(per_event) == 8 * 4  # 8 warps x (2 stores + 2 loads)
        assert all(h["message"] == "shared bank-conflict degree %d" % d and h["degree"] == d for h in per_event)
        assert all(h["severity"] == ("critical" if d >= 8 else "warning") for h in per_event)
        assert any(h["message"] == "32 shared accesses with bank conflicts" for h in hs)
        assert all(info.text(h["pc"]).startswith(("st.shared", "ld.shared")) for h in per_event)


@pytest.mark.parametrize("s", [1, 2, 3, 4, 5, 8, 33])
def test_global_efficiency_hints(A, oracle_mod, s):
    w = W.strided_gather(s, n=512)
    _, (hdr, rec) = ext(oracle_mod, w)
    info = A.ProgramInfo(w.ptx)
    hs = A.hints(hdr, rec, info, warps_per_block=w.warps_per_block)
    # a[i * s]: 32 lanes x 4 bytes fit one line but touch min(32, s) lines
    eff = 1.0 / min(32, s)
    crit = [h for h in hs if h.get("severity") == "critical"]
    if eff < 0.25:
        assert len(crit) == 16 and all(abs(h["efficiency"] - eff) < 1e-12 for h in crit)
        assert all(info.text(h["pc"]).startswith("ld.global") for h in crit)
        assert all(h["message"] == "global access at %d%% coalescing efficiency" % int(eff * 100) for h in crit)
        assert len(hs) == 16
    else:
        # 25-50% is counted as uncoalesced but, as in the rules, gives no hint
        assert hs == []


def test_coalescing_efficiency_page_examples(A, oracle_mod):
    """The memory-analysis part's three global examples, run through the oracle's
    extended records: 32 consecutive words (1 line, efficiency 1.0), a 128-byte
    stride (32 lines, 0.03125) and 32 words from byte 64 (2 lines, 0.5)."""
    from analysis_ptxsimulator_amd import ks
    cases = [([i * 4 for i in range(32)], 1, 1.0), ([i * 128 for i in range(32)], 32, 0.03125),
             ([64 + i * 4 for i in range(32)], 2, 0.5)]
    gaddr = np.concatenate([np.array(c[0], np.uint64) for c in cases])
    w = S.addr_probe(gaddr, np.zeros(len(gaddr), np.uint32), np.ones(len(gaddr), np.uint32), 4096, block=96)
    _, (hdr, rec) = ext(oracle_mod, w)
    info = A.ProgramInfo(w.ptx)
    for wi, (_, lines, eff) in enumerate(cases):
        r = rec[wi, :hdr["records_written"][wi]]
        probe = [x for x in r if int(x["kind"]) == ks.KS_EV_LD_GLOBAL
                 and info.desc[int(x["pc"])]["access_bytes"] == 4 and (int(x["payload"]) >> 8) & 0xFF == lines]
        assert probe, wi
        got = A.coalescing_efficiency(int(probe[0]["kind"]), probe[0]["payload"], 4)
        assert got == eff
    assert A.coalescing_efficiency(ks.KS_EV_OTHER, 0xFFFFFFFF, 4) is None


def test_divergence_and_occupancy_hints(A, oracle_mod):
    # vector_add: warp 31 splits 8 / 24 at the bounds check: ratio 0.25, no warning
    w = W.vector_add()
    _, (hdr, rec) = ext(oracle_mod, w)
    info = A.ProgramInfo(w.ptx)
    assert A.hints(hdr, rec, info, warps_per_block=w.warps_per_block) == []
    # lanes splitting evenly on their data: every divergent branch is a warning
    ptx = S.random_cfg_ptx(3)
    n = 64
    g = np.zeros(8 * n + 4096, np.uint8)
    g[:4 * n] = np.tile(np.array([0, 0xFFFFFFFF], np.uint32), n // 2).view(np.uint8)
    wk = W.Workload(name="cfg", ptx=ptx, grid=(1, 1, 1), block=(n, 1, 1),
                    params=[("param_in", "u64", 0), ("param_out", "u64", 4 * n)], gmem=g, trace_cap=256)
    c, (hdr, rec) = ext(oracle_mod, wk)
    hs = A.hints(hdr, rec, A.ProgramInfo(ptx), warps_per_block=2)
    div = [h for h in hs if h["category"] == "divergence" and "warp" in h]
    n_div = int(c["diverge_n"].sum())
    assert len(div) <= n_div
    for h in div:
        r = rec[h["warp"], h["record"]]
        act, taken = int(r["active"]), int(r["payload"]) & int(r["active"])
        assert min(bin(taken).count("1"), bin(act & ~taken).count("1")) / bin(act).count("1") > 0.4
    if n_div > 3:
        assert any(h["message"] == "%d branches split their warp" % n_div for h in hs)
    assert [h["severity"] for h in A.hints(hdr[:0], rec[:0], info, A.occupancy("sm_80", 256, 32))] == []
    # 25%: not below 25 (no critical), below 50 (warning)
    assert [h["severity"] for h in A.hints(hdr[:0], rec[:0], info, A.occupancy("sm_80", 256, 128))] == ["warning"]
    assert [h["severity"] for h in A.hints(hdr[:0], rec[:0], info, A.occupancy("sm_80", 256, 200))] == ["critical"]
    assert [h["severity"] for h in A.hints(hdr[:0], rec[:0], info, A.occupancy("sm_80", 256, 80))] == ["warning"]


def test_chrome_trace_export(A, oracle_mod):
    w = W.vector_add()
    _, (hdr, rec) = ext(oracle_mod, w)
    info = A.ProgramInfo(w.ptx)
    t = json.loads(json.dumps(A.chrome_trace(hdr, rec, info, w.warps_per_block)))
    gold = json.load(open(os.path.join(GOLDEN, "vector_add_trace.json")))
    cyc = gold["issue_cycles"]
    ev = [e for e in t["traceEvents"] if e["ph"] == "X"]
    assert len(ev) == 32 * 19
    meta = [e for e in t["traceEvents"] if e["ph"] == "M"]
    assert sorted({(e["pid"], e["args"]["name"]) for e in meta if e["name"] == "process_name"}) == \
        [(b, "block %d" % b) for b in range(4)]
    w0 = [e for e in ev if e["pid"] == 0 and e["tid"] == 0]
    assert [e["ts"] for e in w0] == cyc
    assert [e["dur"] for e in w0] == [b - a for a, b in zip(cyc, cyc[1:])] + [1]
    names = [e["name"] for e in w0]
    assert names[:4] == ["ld.param.u64"] * 3 + ["ld.param.u32"]
    assert names[9] == "bra" and names[12] == "ld.global.f32" and names[17] == "st.global.f32" and names[18] == "ret"
    assert w0[12]["args"]["sectors"] == 4 and w0[12]["args"]["lines"] == 1 and w0[12]["cat"] == "ld.global"
    w31 = [e for e in ev if e["pid"] == 3 and e["tid"] == 7]
    assert w31[9]["cat"] == "diverge" and w31[9]["args"]["taken"] == 0xFFFFFF00
    assert w31[12]["args"]["active"] == "0x000000ff"
    # the basic 8-byte records export the same timeline, without payloads
    g = w.gmem.copy()
    _, tb, _ = oracle_mod.run(w.ptx, w.grid, w.block, w.params_bytes, g, trace_cap=w.trace_cap)
    hb, rb = oracle_mod.trace_slots(tb, w.trace_cap)
    tbj = A.chrome_trace(hb, rb, info, w.warps_per_block, trace_format=0)
    evb = [e for e in tbj["traceEvents"] if e["ph"] == "X"]
    assert [(e["ts"], e["dur"], e["name"]) for e in evb] == [(e["ts"], e["dur"], e["name"]) for e in ev]


def _random_ext(O, seed=4, grid=2, block=64, cap=512):
    w = W.random_stress(prog_seed=seed, grid=grid, block=block, gmem_bytes=1 << 16, n_instr=300, trace_cap=cap)
    _, (hdr, rec) = ext(O, w)
    return w, hdr, rec


@pytest.mark.parametrize("seed", [4, 11])
def test_hint_table_matches_a_record_by_record_pass(A, oracle_mod, seed):
    """The array pass of hint_table against the rules applied to one record at a
    time (pure Python over the decoded fields)."""
    from analysis_ptxsimulator_amd import ks
    w, hdr, rec = _random_ext(oracle_mod, seed)
    info = A.ProgramInfo(w.ptx)
    t = A.hint_table(hdr, rec, info)
    want, conflicts, unco, divergent = [], 0, 0, 0
    popc = lambda x: bin(x & 0xFFFFFFFF).count("1")
    for wi in range(len(hdr)):
        for k in range(int(hdr["records_written"][wi])):
            r = rec[wi, k]
            kind, pc, act, pay = int(r["kind"]), int(r["pc"]), int(r["active"]), int(r["payload"])
            if kind in (ks.KS_EV_LD_SHARED, ks.KS_EV_ST_SHARED) and (pay & 0xFF) > 1:
                conflicts += 1
                want.append((wi, k, pc, 0, float(pay & 0xFF)))
            elif kind in (ks.KS_EV_LD_GLOBAL, ks.KS_EV_ST_GLOBAL) and (pay >> 8) & 0xFF:
                lanes, lines = (pay >> 16) & 0xFF, (pay >> 8) & 0xFF
                eff = min(1.0, -(-lanes * info.desc[pc]["access_bytes"] // 128) / lines)
                if eff < 0.25:
                    want.append((wi, k, pc, 1, eff))
                elif eff < 0.5:
                    unco += 1
            elif kind == ks.KS_EV_DIVERGE:
                divergent += 1
                tk = pay & act
                ratio = min(popc(tk), popc(act & ~tk)) / max(1, popc(act))
                if ratio > 0.4:
                    want.append((wi, k, pc, 2, ratio))
    got = list(zip(t["warp"].tolist(), t["record"].tolist(), t["pc"].tolist(), t["rule"].tolist(),
                   t["value"].tolist()))
    assert got == want
    assert (t["conflicts"], t["uncoalesced"], t["divergent"]) == (conflicts, unco, divergent)
    assert len(want) > 0 and t["conflicts"] + t["divergent"] > 0


def test_trace_export_matches_the_records(A, oracle_mod):
    """Every field of every event of the native export against the records it
    came from: block/warp metadata before each warp's events, durations to the
    warp's next issue, payload fields by kind."""
    from analysis_ptxsimulator_amd import ks
    w, hdr, rec = _random_ext(oracle_mod, 7, grid=3, block=96)
    info = A.ProgramInfo(w.ptx)
    wpb = w.warps_per_block
    t = A.chrome_trace(hdr, rec, info, wpb)
    want = []
    for wi in range(len(hdr)):
        n = int(hdr["records_written"][wi])
        if not n:
            continue
        b, wib = wi // wpb, wi % wpb
        if wib == 0:
            want.append({"ph": "M", "name": "process_name", "pid": b, "tid": 0, "args": {"name": "block %d" % b}})
        want.append({"ph": "M", "name": "thread_name", "pid": b, "tid": wib, "args": {"name": "warp %d" % wib}})
        for k in range(n):
            r = rec[wi, k]
            pc, kind, act, pay = int(r["pc"]), int(r["kind"]), int(r["active"]), int(r["payload"])
            cyc = int(r["cycle"])
            dur = int(rec[wi, k + 1]["cycle"]) - cyc if k + 1 < n else 1
            args = {"pc": pc, "line": info.desc[pc]["line"], "text": info.text(pc), "active": "0x%08x" % act}
            if kind in (ks.KS_EV_LD_GLOBAL, ks.KS_EV_ST_GLOBAL):
                args.update(sectors=pay & 0xFF, lines=(pay >> 8) & 0xFF, lanes=(pay >> 16) & 0xFF, faults=pay >> 24)
            elif kind in (ks.KS_EV_LD_SHARED, ks.KS_EV_ST_SHARED):
                args.update(degree=pay & 0xFF, lanes=(pay >> 16) & 0xFF, faults=pay >> 24)
            elif kind in (ks.KS_EV_BRANCH, ks.KS_EV_DIVERGE):
                args.update(taken=pay)
            elif kind != ks.KS_EV_BARRIER:
                args.update(guard_lanes=pay)
            want.append({"ph": "X", "name": info.mnemonic(pc), "cat": ks.EV_NAMES[kind], "pid": b, "tid": wib,
                         "ts": cyc, "dur": dur, "args": args})
    assert t["traceEvents"] == want
    assert t["otherData"]["time_unit"] == "simulated cycle"
    # a slice of warps keeps its global numbering
    t2 = A.chrome_trace(hdr[wpb:], rec[wpb:], info, wpb, first_warp=wpb)
    assert t2["traceEvents"] == [e for e in want if e["pid"] >= 1]


def test_trace_export_rejects_records_outside_the_program(A, oracle_mod, tmp_path):
    from analysis_ptxsimulator_amd import ks
    w, hdr, rec = _random_ext(oracle_mod, 7)
    info = A.ProgramInfo(w.ptx)
    bad = rec.copy()
    bad[0, 0]["pc"] = len(info.desc)
    with pytest.raises(ks.KsError, match="outside the program"):
        A.write_chrome_trace(str(tmp_path / "t.json"), hdr, bad, info, w.warps_per_block)
    h2 = hdr.copy()
    h2["records_written"][0] = rec.shape[1] + 1
    with pytest.raises(ks.KsError, match="records in a slot"):
        A.write_chrome_trace(str(tmp_path / "t.json"), h2, rec, info, w.warps_per_block)
    with pytest.raises(ks.KsError, match="cannot open"):
        A.write_chrome_trace(str(tmp_path / "no" / "t.json"), hdr, rec, info, w.warps_per_block)
    raw = A._slot_bytes(hdr, rec, ks.KS_TRACE_EXTENDED)
    names = (ctypes.c_char_p * len(info.desc))(*([b'"x"'] * (len(info.desc) - 1) + [None]))
    args = (ctypes.c_char_p * len(info.desc))(*([b'"pc":0'] * len(info.desc)))
    rc = ks.lib().ks_write_trace_events(raw.ctypes.data_as(ctypes.c_void_p), len(hdr), raw.shape[1],
                                        ks.KS_TRACE_EXTENDED, 0, w.warps_per_block, len(info.desc), names, args,
                                        str(tmp_path / "t.json").encode(), None)
    assert rc == -3 and b"NULL name" in ks.lib().ks_last_error()  # KS_E_INVALID_ARG
    n = A.write_chrome_trace(str(tmp_path / "t.json"), hdr, rec, info, w.warps_per_block)
    assert n == int(hdr["records_written"].sum())


def test_param_block_uses_the_library_layout(A):
    """param_block packs named values at the offsets the library reads: vector_add's
    block equals the workload's own packing; floats are binary32; unnamed
    parameters are 0; an unknown name or an oversized value is refused."""
    import struct
    vals = {"param_a": 0, "param_b": 4096, "param_c": 8192, "param_n": 1000}
    assert A.param_block(W.VECTOR_ADD_PTX, vals) == W.vector_add().params_bytes
    b = A.param_block(W.VECTOR_ADD_PTX, {"param_c": 0x1234, "param_n": 1.5})
    assert b[16:24] == (0x1234).to_bytes(8, "little") and b[24:28] == struct.pack("<f", 1.5) and b[:16] == bytes(16)
    assert A.param_block(W.VECTOR_ADD_PTX, {"param_n": -1})[24:28] == b"\xff\xff\xff\xff"
    with pytest.raises(ValueError, match="no parameter named param_x"):
        A.param_block(W.VECTOR_ADD_PTX, {"param_x": 1})
    with pytest.raises(ValueError, match="does not fit"):
        A.param_block(W.VECTOR_ADD_PTX, {"param_n": 1 << 32})
    with pytest.raises(ValueError, match="a float needs 4"):
        A.param_block(W.VECTOR_ADD_PTX, {"param_a": 0.5})
    with pytest.raises(ValueError, match="beyond binary32"):
        A.param_block(W.VECTOR_ADD_PTX, {"param_n": 1e39})
    with pytest.raises(SystemExit, match="comma-separated integers"):
        A._dims("4,x")


@pytest.mark.parametrize("pad", [0, 1])
def test_transpose_bank_conflict_hint(A, oracle_mod, pad):
    """On the shared-tile transpose the hint rules flag the unpadded tile's column
    load (degree 32, critical) in every warp, and nothing once the tile is padded."""
    gx = 2
    n = 32 * gx
    g = np.zeros(8 * n * n, np.uint8)
    g[:4 * n * n] = np.arange(n * n, dtype=np.uint32).view(np.uint8)
    w = W.Workload(name="tile_transpose", ptx=S.tile_transpose_ptx(pad), grid=(gx, gx, 1), block=(32, 32, 1),
                   params=[("param_in", "u64", 0), ("param_out", "u64", 4 * n * n)], gmem=g, trace_cap=64)
    _, (hdr, rec) = ext(oracle_mod, w)
    info = A.ProgramInfo(w.ptx)
    hs = A.hints(hdr, rec, info, warps_per_block=w.warps_per_block)
    per_event = [h for h in hs if "warp" in h and "bank-conflict degree" in h["message"]]
    if pad:
        assert per_event == []
    else:
        assert len(per_event) == w.n_warps
        assert all(h["degree"] == 32 and h["severity"] == "critical" for h in per_event)
        assert all(info.text(h["pc"]).startswith("ld.shared") for h in per_event)
