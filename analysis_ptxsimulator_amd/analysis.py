"""Host analysis of the simulator's outputs: occupancy, hints and a timeline export.

Post-processing of what a ks_run leaves behind (per-warp counters and trace
slots, best with extended records); nothing here simulates.

* Occupancy: the KernelScope occupancy-calculator model (KernelScope backend
  documentation, github.com/briefgaming/kernelscope, "occupancy/calculator.py"
  part): active warps per SM limited by registers (allocated per warp in groups
  of 256), by shared memory (allocated per block in 256-byte chunks) and by the
  block limits (threads per SM, blocks per SM); occupancy = active / max warps.
* Hints: the rules of the same documentation's "hints/analyzer.py" part, applied
  to extended trace records: a shared access with a conflict degree of 8 or more
  is critical and one above 1 a warning; a global access with less than 25%
  coalescing efficiency (memory-analysis part: ideal over touched 128-byte lines)
  is critical, one below 50% counts as uncoalesced; a divergent branch
  whose divergence ratio exceeds 40% is a warning; more than 5 conflicting shared
  accesses or more than 3 divergent branches give a summary warning; occupancy
  below 25% is critical and below 50% a warning.
* Timeline: the per-warp slots exported as a Chrome trace-event file (loadable in
  Perfetto), the "postprocess -> Perfetto trace" step of the IKET page ("CuTeDSL
  IKET 浅析", zhen8838.github.io/posts/iket.html, sections 3 and 5).
"""
import json
import re

import numpy as np

from . import ks

# Per-architecture limits of the occupancy model.  sm_75 and sm_80 are given in full
# on the KernelScope page; for sm_86, sm_89 and sm_90 it elides some fields, which
# take NVIDIA's published values (64K registers per SM throughout; 100 KB of shared
# memory per SM for sm_86 and sm_89).
GPU_SPECS = {
    "sm_75": dict(name="Turing (T4)", max_threads_per_sm=1024, max_warps_per_sm=32, max_blocks_per_sm=16,
                  max_threads_per_block=1024, registers_per_sm=65536, max_registers_per_thread=255,
                  shared_memory_per_sm=65536, max_shared_memory_per_block=49152),
    "sm_80": dict(name="Ampere (A100)", max_threads_per_sm=2048, max_warps_per_sm=64, max_blocks_per_sm=32,
                  max_threads_per_block=1024, registers_per_sm=65536, max_registers_per_thread=255,
                  shared_memory_per_sm=167936, max_shared_memory_per_block=163840),
    "sm_86": dict(name="Ampere (RTX 3090)", max_threads_per_sm=1536, max_warps_per_sm=48, max_blocks_per_sm=16,
                  max_threads_per_block=1024, registers_per_sm=65536, max_registers_per_thread=255,
                  shared_memory_per_sm=102400, max_shared_memory_per_block=101376),
    "sm_89": dict(name="Ada (RTX 4090)", max_threads_per_sm=1536, max_warps_per_sm=48, max_blocks_per_sm=24,
                  max_threads_per_block=1024, registers_per_sm=65536, max_registers_per_thread=255,
                  shared_memory_per_sm=102400, max_shared_memory_per_block=101376),
    "sm_90": dict(name="Hopper (H100)", max_threads_per_sm=2048, max_warps_per_sm=64, max_blocks_per_sm=32,
                  max_threads_per_block=1024, registers_per_sm=65536, max_registers_per_thread=255,
                  shared_memory_per_sm=232448, max_shared_memory_per_block=232448),
}


def _round_up(x, g):
    return (x + g - 1) // g * g


def occupancy(arch, threads_per_block, registers_per_thread, shared_bytes_per_block=0):
    """Active warps per SM and the occupancy of a launch shape (the three limiters of
    the occupancy model; ties name registers first, then shared memory)."""
    spec = GPU_SPECS[arch]
    if not 1 <= threads_per_block <= spec["max_threads_per_block"]:
        raise ValueError("block of %d threads on %s" % (threads_per_block, arch))
    wpb = (threads_per_block + 31) // 32
    maxw = spec["max_warps_per_sm"]
    if registers_per_thread > 0:
        per_warp = _round_up(registers_per_thread * 32, 256)
        by_regs = spec["registers_per_sm"] // per_warp
    else:
        by_regs = maxw
    if shared_bytes_per_block > 0:
        by_smem = (spec["shared_memory_per_sm"] // _round_up(shared_bytes_per_block, 256)) * wpb
    else:
        by_smem = maxw
    blocks = min(spec["max_threads_per_sm"] // threads_per_block, spec["max_blocks_per_sm"])
    by_block = blocks * wpb
    active = min(by_regs, by_smem, by_block, maxw)
    limiter = "registers" if active == by_regs else ("shared_memory" if active == by_smem else "block_size")
    return {"arch": arch, "active_warps_per_sm": active, "max_warps_per_sm": maxw,
            "occupancy_percent": 100.0 * active / maxw, "limiting_factor": limiter,
            "warps_by_registers": by_regs, "warps_by_shared_memory": by_smem, "warps_by_block_size": by_block}


def program_occupancy(ptx, block_threads, arch="sm_80"):
    """Occupancy of a simulated program: its declared 32-bit register slots per
    thread (a 64-bit register counts two) and its .shared bytes per block."""
    prog = ks.ks_load_program(ptx)
    try:
        info = ks.ks_program_info(prog)
    finally:
        ks.ks_program_free(prog)
    return occupancy(arch, block_threads, info["reg_slots"], info["shared_bytes"])


class ProgramInfo:
    """pc -> (source line, text, access bytes) of a program, from ks_instr_info."""

    def __init__(self, ptx):
        self.lines = ptx.split("\n")
        prog = ks.ks_load_program(ptx)
        try:
            n = ks.ks_program_info(prog)["n_instrs"]
            self.desc = [ks.ks_instr_info(prog, pc) for pc in range(n)]
        finally:
            ks.ks_program_free(prog)

    def text(self, pc):
        t = self.lines[self.desc[pc]["line"] - 1].strip()
        return re.sub(r"\s*//.*$", "", t).rstrip(";").strip()

    def mnemonic(self, pc):
        return re.sub(r"^@!?%\w+\s+", "", self.text(pc)).split()[0]


def decode_payload(kind, payload):
    """Fields of an extended record's payload (see include/ks.h)."""
    p = int(payload)
    if kind in (ks.KS_EV_LD_GLOBAL, ks.KS_EV_ST_GLOBAL):
        return {"sectors": p & 0xFF, "lines": (p >> 8) & 0xFF, "lanes": (p >> 16) & 0xFF, "faults": p >> 24}
    if kind in (ks.KS_EV_LD_SHARED, ks.KS_EV_ST_SHARED):
        return {"degree": p & 0xFF, "lanes": (p >> 16) & 0xFF, "faults": p >> 24}
    if kind in (ks.KS_EV_BRANCH, ks.KS_EV_DIVERGE):
        return {"taken": p}
    if kind == ks.KS_EV_BARRIER:
        return {}
    return {"guard_lanes": p}


def _popc(x):
    return bin(int(x)).count("1")


def coalescing_efficiency(kind, payload, access_bytes):
    """Efficiency of a global access record (KernelScope memory-analysis part):
    the whole 128-byte lines its requested bytes need, over the lines it touches,
    at most 1; None for other records or an access with no guard lane."""
    if kind not in (ks.KS_EV_LD_GLOBAL, ks.KS_EV_ST_GLOBAL):
        return None
    f = decode_payload(kind, payload)
    if not f["lines"]:
        return None
    return min(1.0, ((f["lanes"] * access_bytes + 127) // 128) / f["lines"])


def hints(headers, records, info, occupancy_result=None, warps_per_block=1):
    """The hint rules over extended trace records (one slot per warp).  Per-event
    hints carry the warp, the record index, the pc and the source line.

    The efficiency of a global access is the coalescing analysis's: the fewest
    128-byte lines its requested bytes could take (guard lanes x access bytes,
    rounded up to whole lines) over the lines it touches, at most 1.  Accesses
    between 25% and 50% are counted as uncoalesced but, as in the rules, produce
    no hint.  Reading (the rules use a ratio they do not define): the divergence
    ratio of a divergent branch = lanes on the smaller side / active lanes (0.5
    for an even split)."""
    out = []
    n_conflict = n_uncoalesced = n_divergent = 0
    for w in range(len(headers)):
        n = int(headers["records_written"][w])
        for k in range(n):
            r = records[w, k]
            kind, pc = int(r["kind"]), int(r["pc"])
            where = {"warp": w, "block": w // warps_per_block, "record": k, "pc": pc,
                     "source_line": info.desc[pc]["line"]}
            f = decode_payload(kind, r["payload"])
            if kind in (ks.KS_EV_LD_SHARED, ks.KS_EV_ST_SHARED) and f["degree"] > 1:
                n_conflict += 1
                sev = "critical" if f["degree"] >= 8 else "warning"
                out.append(dict(category="memory", severity=sev, message="%d-way bank conflict" % f["degree"],
                                detail="Severe bank conflict causing serialized access" if sev == "critical"
                                else "Bank conflict reducing throughput", **where))
            elif kind in (ks.KS_EV_LD_GLOBAL, ks.KS_EV_ST_GLOBAL) and f["lines"]:
                eff = coalescing_efficiency(kind, r["payload"], info.desc[pc]["access_bytes"])
                if eff < 0.25:
                    out.append(dict(category="memory", severity="critical",
                                    message="Poor memory efficiency (%d%%)" % int(eff * 100),
                                    detail="Scattered access causing many transactions", efficiency=eff, **where))
                elif eff < 0.5:
                    n_uncoalesced += 1
            elif kind == ks.KS_EV_DIVERGE:
                n_divergent += 1
                act, taken = int(r["active"]), f["taken"] & int(r["active"])
                ratio = min(_popc(taken), _popc(act & ~taken)) / max(1, _popc(act))
                if ratio > 0.4:
                    out.append(dict(category="divergence", severity="warning",
                                    message="High divergence (%d%%)" % int(ratio * 100),
                                    detail="Significant warp divergence at this branch", ratio=ratio, **where))
    if n_conflict > 5:
        out.append(dict(category="memory", severity="warning",
                        message="Shared memory bank conflicts (%d events)" % n_conflict,
                        detail="Consider padding arrays or restructuring access patterns"))
    if n_divergent > 3:
        out.append(dict(category="divergence", severity="warning",
                        message="Branch divergence detected (%d events)" % n_divergent,
                        detail="Consider restructuring conditionals or using predication"))
    if occupancy_result:
        occ, lim = occupancy_result["occupancy_percent"], occupancy_result["limiting_factor"]
        if occ < 25:
            out.append(dict(category="occupancy", severity="critical", message="Very low occupancy (%g%%)" % occ,
                            detail="Limited by %s. Consider reducing resource usage." % lim))
        elif occ < 50:
            out.append(dict(category="occupancy", severity="warning", message="Low occupancy (%g%%)" % occ,
                            detail="Limited by %s." % lim))
    return out


def chrome_trace(headers, records, info, warps_per_block, trace_format=ks.KS_TRACE_EXTENDED):
    """Trace-event JSON of the per-warp slots: one process per block, one thread per
    warp, one complete event per issued instruction from its issue cycle to the
    warp's next issue (1 cycle for the last).  Time unit: one simulated cycle."""
    ev = []
    for w in range(len(headers)):
        n = int(headers["records_written"][w])
        if n == 0:
            continue
        b, wib = w // warps_per_block, w % warps_per_block
        if wib == 0:
            ev.append({"ph": "M", "name": "process_name", "pid": b, "tid": 0, "args": {"name": "block %d" % b}})
        ev.append({"ph": "M", "name": "thread_name", "pid": b, "tid": wib, "args": {"name": "warp %d" % wib}})
        if trace_format == ks.KS_TRACE_EXTENDED:
            cyc = records[w, :n]["cycle"].astype(np.int64)
            pcs = records[w, :n]["pc"].astype(np.int64)
        else:
            cyc = records[w, :n, 0].astype(np.int64)
            pcs = records[w, :n, 1].astype(np.int64)
        for k in range(n):
            pc = int(pcs[k])
            dur = int(cyc[k + 1] - cyc[k]) if k + 1 < n else 1
            args = {"pc": pc, "line": info.desc[pc]["line"], "text": info.text(pc)}
            cat = "issue"
            if trace_format == ks.KS_TRACE_EXTENDED:
                r = records[w, k]
                kind = int(r["kind"])
                cat = ks.EV_NAMES[kind]
                args["active"] = "0x%08x" % int(r["active"])
                args.update(decode_payload(kind, r["payload"]))
            ev.append({"ph": "X", "name": info.mnemonic(pc), "cat": cat, "pid": b, "tid": wib,
                       "ts": int(cyc[k]), "dur": dur, "args": args})
    return {"traceEvents": ev, "displayTimeUnit": "ns",
            "otherData": {"time_unit": "simulated cycle", "source": "libkscope per-warp trace slots"}}


def main(argv=None):
    """Run a workload on the GPU with extended records and report occupancy, hints
    and (with --out) a Chrome/Perfetto trace of its first warps."""
    import argparse
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import configs as W
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="vector_add",
                    help="vector_add | strided_<s> | bank_<s> | ffma_<acc> | random_<seed>")
    ap.add_argument("--arch", default="sm_80")
    ap.add_argument("--out", default=None, help="write the trace-event JSON here")
    ap.add_argument("--warps", type=int, default=64, help="warps exported to the timeline")
    args = ap.parse_args(argv)
    name = args.workload
    if name == "vector_add":
        w = W.vector_add()
    elif name.startswith("strided_"):
        w = W.strided_gather(int(name[8:]), n=8192)
    elif name.startswith("bank_"):
        w = W.bank_probe(int(name[5:]), iters=16, grid=8, block=1024, trace_cap=128)
    elif name.startswith("ffma_"):
        w = W.ffma_probe(int(name[5:]), iters=64, grid=8, block=256, trace_cap=4096)
    elif name.startswith("random_"):
        w = W.random_stress(prog_seed=int(name[7:]), grid=16, block=256, gmem_bytes=1 << 24, trace_cap=2048)
    else:
        raise SystemExit("unknown workload %s" % name)
    s = ks.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=w.trace_cap, trace_format=ks.KS_TRACE_EXTENDED)
    try:
        s.load_gmem(w.gmem)
        s.run(w.params_bytes)
        hdr, rec = s.trace_records()
        kernel = s.kernel_name()
    finally:
        s.close()
    info = ProgramInfo(w.ptx)
    occ = program_occupancy(w.ptx, w.threads_per_block, args.arch)
    hs = hints(hdr, rec, info, occ, w.warps_per_block)
    print(json.dumps({"workload": w.name, "kernel": kernel, "occupancy": occ,
                      "hints": [h for h in hs if "warp" not in h] + [h for h in hs if "warp" in h][:20],
                      "n_event_hints": sum(1 for h in hs if "warp" in h)}, indent=1))
    if args.out:
        with open(args.out, "w") as f:
            json.dump(chrome_trace(hdr[: args.warps], rec[: args.warps], info, w.warps_per_block), f)


if __name__ == "__main__":
    main()
