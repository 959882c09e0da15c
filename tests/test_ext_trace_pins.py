"""Pins of the extended (16-byte) trace records on the CPU oracle.

The extended record is the IKET page's "event with a payload" shape (section 2:
16-byte events once a payload is carried) filled with what the KernelScope pages
attach to an instruction: its kind (memory access, branch, divergence, barrier),
the warp's active mask, and the memory analysis of the access or the lanes taking
the branch.  Pinned here by:

* the vector_add listing, record by record, derived by hand (kinds, masks,
  payloads; issue cycles from the existing hand derivation in tests/golden);
* the closed forms of the strided and bank probes, now per access;
* invariants that tie every record field to the per-warp counters, which the
  oracle computes separately, and to the basic 8-byte trace of the same run.
"""
import json
import math
import os

import numpy as np
import pytest

from workloads import configs as W
from workloads import probes as PR
from workloads import small as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
OTHER, LDG, STG, LDS, STS, BRANCH, DIVERGE, BARRIER, RET = range(9)


def ext_run(O, w, cap=None, **kw):
    cap = w.trace_cap if cap is None else cap
    g = w.gmem.copy()
    c, t, _ = O.run(w.ptx, w.grid, w.block, w.params_bytes, g, trace_cap=cap, trace_format=O.TRACE_EXTENDED, **kw)
    hdr, rec = O.trace_slots(t, cap, O.TRACE_EXTENDED)
    return g, c, hdr, rec


def popc(x):
    return bin(int(x)).count("1")


def test_vector_add_records_by_hand(oracle_mod):
    w = W.vector_add()
    _, c, hdr, rec = ext_run(oracle_mod, w)
    gold = json.load(open(os.path.join(GOLDEN, "vector_add_trace.json")))
    kinds = [OTHER] * 9 + [BRANCH, OTHER, OTHER, LDG, OTHER, LDG, OTHER, OTHER, STG, RET]
    full = 0xFFFFFFFF
    coalesced = 4 | (1 << 8) | (32 << 16)    # 32 lanes x 4 bytes: 4 sectors, 1 line
    for wi in range(32):
        r = rec[wi, :hdr["records_written"][wi]]
        assert hdr["version"][wi] == 2 and hdr["records_written"][wi] == 19
        assert list(r["pc"]) == list(range(19))
        assert list(r["cycle"]) == gold["issue_cycles"]
        assert (r["reserved"] == 0).all()
        if wi < 31:
            assert list(r["kind"]) == kinds
            assert (r["active"] == full).all()
            for k, (kind, pay) in enumerate(zip(r["kind"], r["payload"])):
                want = {BRANCH: 0, LDG: coalesced, STG: coalesced}.get(int(kind), full)
                assert pay == want, (wi, k)
        else:
            # warp 31 holds threads 992..1023 of n = 1000: lanes 8..31 take the exit
            # branch, lanes 0..7 run the body (fall-through first), all meet at ret
            k31 = list(kinds)
            k31[9] = DIVERGE
            assert list(r["kind"]) == k31
            assert list(r["active"]) == [full] * 10 + [0xFF] * 8 + [full]
            assert r["payload"][9] == 0xFFFFFF00
            for k in (12, 14, 17):
                assert r["payload"][k] == 1 | (1 << 8) | (8 << 16)  # 8 lanes x 4 bytes: 1 sector
            for k in (10, 11, 13, 15, 16):
                assert r["payload"][k] == 0xFF
            assert r["payload"][18] == full
    assert c["diverge_n"][31] == 1 and (c["diverge_n"][:31] == 0).all()


def _check_against_counters(c, hdr, rec):
    """Every counter that the records can express equals the records' sum."""
    for wi in range(len(c)):
        n = int(hdr["records_written"][wi])
        assert n == c["warp_instrs"][wi] and hdr["records_dropped"][wi] == 0
        r = rec[wi, :n]
        kind, pay, act = r["kind"].astype(int), r["payload"].astype(np.int64), r["active"]
        assert np.all(np.diff(r["cycle"].astype(np.int64)) >= 1)
        assert sum(popc(a) for a in act) == c["thread_instrs"][wi]
        for k_ld, prefix in ((LDG, "gld"), (STG, "gst")):
            sel = kind == k_ld
            lanes = (pay[sel] >> 16) & 0xFF
            assert int(np.sum(pay[sel] & 0xFF)) == c[prefix + "_sectors"][wi]
            assert int(np.sum((pay[sel] >> 8) & 0xFF)) == c[prefix + "_lines"][wi]
            assert int(np.sum(lanes > 0)) == c[prefix + "_n"][wi]
            # a guard lane count equals the popcount of the guard-passing active lanes
            assert np.all(lanes <= np.array([popc(a) for a in act[sel]], dtype=np.int64))
        sh = (kind == LDS) | (kind == STS)
        deg = pay[sh] & 0xFF
        assert int(np.sum(deg)) == c["sh_degree_sum"][wi]
        assert int(deg.max(initial=0)) == c["sh_degree_max"][wi]
        assert int(np.sum(deg > 0)) == c["sh_n"][wi]
        mem = (kind >= LDG) & (kind <= STS)
        assert int(np.sum((pay[mem] >> 24) & 0xFF)) == c["fault_n"][wi]
        assert int(np.sum(kind == DIVERGE)) == c["diverge_n"][wi]
        assert int(np.sum(kind == BARRIER)) == c["barrier_n"][wi]
        br = (kind == BRANCH) | (kind == DIVERGE)
        # a branch diverges exactly when some but not all active lanes take it
        for a, p, k in zip(act[br], pay[br], kind[br]):
            assert (int(p) & ~int(a)) == 0
            assert (k == DIVERGE) == (0 < (int(p) & int(a)) != int(a))
        other = (kind == OTHER) | (kind == RET)
        assert np.all((r["payload"][other] & ~r["active"][other]) == 0)


def _workloads():
    return [W.vector_add(), W.strided_gather(3, n=2048), W.ffma_probe(3, iters=3, grid=2, block=64, trace_cap=512),
            W.bank_probe(12, iters=3, grid=2, block=256, trace_cap=64),
            W.random_stress(prog_seed=1, grid=4, block=128, gmem_bytes=1 << 22, trace_cap=4096),
            PR.chain_probe("mad.s32", 3, 4, grid=2, block=40, trace_cap=256)]


@pytest.mark.parametrize("k", range(6))
def test_records_agree_with_counters_and_basic_trace(oracle_mod, k):
    w = _workloads()[k]
    g, c, hdr, rec = ext_run(oracle_mod, w)
    _check_against_counters(c, hdr, rec)
    gb = w.gmem.copy()
    cb, tb, _ = oracle_mod.run(w.ptx, w.grid, w.block, w.params_bytes, gb, trace_cap=w.trace_cap)
    hb, rb = oracle_mod.trace_slots(tb, w.trace_cap)
    assert np.array_equal(g, gb)
    assert np.array_equal(c, cb)
    assert np.array_equal(hb["records_written"], hdr["records_written"]) and (hb["version"] == 1).all()
    for wi in range(len(c)):
        n = int(hdr["records_written"][wi])
        assert np.array_equal(rb[wi, :n, 0], rec[wi, :n]["cycle"])
        assert np.array_equal(rb[wi, :n, 1], rec[wi, :n]["pc"].astype(np.uint32))


def test_faulting_lanes_in_payload(oracle_mod):
    data = 1 << 16
    gaddr = np.array([0, 2, 30, data + 64] + [0] * 28, np.uint64)
    guard = np.array([1, 1, 1, 1] + [0] * 28, np.uint32)
    w = S.addr_probe(gaddr, np.zeros(32, np.uint32), guard, data, block=32)
    _, c, hdr, rec = ext_run(oracle_mod, w)
    r = rec[0, :hdr["records_written"][0]]
    ldg = r[r["kind"] == LDG]
    # the address-vector load plus the probed load; the probed one has 4 guard lanes, 2 faulting
    probe = [int(p) for p in ldg["payload"] if (int(p) >> 16) & 0xFF == 4]
    assert probe == [len({0, 1, (data + 64) // 32}) | (len({0, (data + 64) // 128}) << 8) | (4 << 16) | (2 << 24)]
    _check_against_counters(c, hdr, rec)


@pytest.mark.parametrize("s", W.STRIDES)
def test_strided_payload_closed_form(oracle_mod, s):
    w = W.strided_gather(s, n=1024)
    _, c, hdr, rec = ext_run(oracle_mod, w)
    for wi in range(len(c)):
        r = rec[wi, :hdr["records_written"][wi]]
        loads = r[r["kind"] == LDG]["payload"]
        assert len(loads) == 2
        assert int(loads[0]) == min(32, 4 * s) | (min(32, s) << 8) | (32 << 16)  # a[i * s]
        assert int(loads[1]) == 4 | (1 << 8) | (32 << 16)                     # b[i]


@pytest.mark.parametrize("s", [1, 2, 3, 8, 24, 32])
def test_bank_degree_in_every_shared_record(oracle_mod, s):
    w = W.bank_probe(s, iters=2, grid=1, block=256, trace_cap=64)
    _, c, hdr, rec = ext_run(oracle_mod, w)
    for wi in range(len(c)):
        r = rec[wi, :hdr["records_written"][wi]]
        sh = r[(r["kind"] == LDS) | (r["kind"] == STS)]
        assert len(sh) == 4
        assert all(int(p) == math.gcd(s, 32) | (32 << 16) for p in sh["payload"])
        assert int(np.sum(r["kind"] == BARRIER)) == 2
