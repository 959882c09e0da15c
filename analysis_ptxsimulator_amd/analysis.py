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


def program_occupancy(ptx, block_threads, arch="sm_80", entry=None):
    """Occupancy of a simulated program: its declared 32-bit register slots per
    thread (a 64-bit register counts two) and its .shared bytes per block."""
    prog = ks.ks_load_program(ptx, entry)
    try:
        info = ks.ks_program_info(prog)
    finally:
        ks.ks_program_free(prog)
    return occupancy(arch, block_threads, info["reg_slots"], info["shared_bytes"])


class ProgramInfo:
    """pc -> (source line, text, access bytes) of a program, from ks_instr_info."""

    def __init__(self, ptx, entry=None):
        self.lines = ptx.split("\n")
        prog = ks.ks_load_program(ptx, entry)
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


def _popc32(x):
    """Per-element population count of a uint32 array."""
    x = np.asarray(x, dtype=np.uint32)
    return np.unpackbits(x.view(np.uint8).reshape(x.shape + (4,)), axis=-1).sum(axis=-1, dtype=np.int64)


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


# Thresholds of the hint rules (KernelScope "hints/analyzer.py" part): a shared access
# whose conflict degree reaches 8 is critical, above 1 a warning; a global access
# below 25% efficiency is critical, below 50% uncoalesced (counted, no event hint);
# a divergent branch whose divergence ratio exceeds 40% is a warning; more than 5
# conflicting shared accesses or more than 3 divergent branches add a summary
# warning; occupancy below 25% is critical, below 50% a warning.
RULES = dict(degree_critical=8, efficiency_critical=0.25, efficiency_uncoalesced=0.5, divergence_ratio=0.4,
             conflicts_summary=5, divergent_summary=3, occupancy_critical=25.0, occupancy_warning=50.0)


def hint_table(headers, records, info):
    """The per-record measures the hint rules look at, over every written extended
    record at once (numpy arrays over [warp, record] positions).

    Returns a dict of flat arrays for the records that trip a rule: `warp`,
    `record`, `pc`, `rule` (0 shared conflict, 1 scattered global access, 2 split
    branch), `value` (conflict degree, coalescing efficiency or divergence ratio),
    plus the totals `conflicts` (shared accesses with a degree above 1),
    `uncoalesced` (global accesses at 25-50% efficiency) and `divergent`
    (divergent branches).

    Efficiency of a global access: the fewest 128-byte lines its requested bytes
    need (guard lanes x access bytes, rounded up to whole lines) over the lines it
    touches, at most 1.  Divergence ratio (the rules use it without defining it;
    reading): lanes on the smaller side of the split over the live lanes."""
    n_w = len(headers)
    cap = records.shape[1] if records.ndim == 2 else 0
    written = np.asarray(headers["records_written"], dtype=np.int64).reshape(n_w)
    # the 16-byte records as four words: cycle, pc | kind << 16, active, payload
    words = np.ascontiguousarray(records).view(np.uint32).reshape(n_w, cap, 4)
    pk = words[:, :, 1]
    kind = (pk >> 16) & 0xFF
    live = np.arange(cap, dtype=np.int64)[None, :] < written[:, None]
    kind = np.where(live, kind, 0xFF)  # unwritten positions take a kind no rule looks at
    pay = words[:, :, 3]
    deg = pay & 0xFF
    conflict = ((kind == ks.KS_EV_LD_SHARED) | (kind == ks.KS_EV_ST_SHARED)) & (deg > 1)
    glob = ((kind == ks.KS_EV_LD_GLOBAL) | (kind == ks.KS_EV_ST_GLOBAL)) & (((pay >> 8) & 0xFF) > 0)
    div = kind == ks.KS_EV_DIVERGE
    acc = np.array([d["access_bytes"] for d in info.desc] + [0], dtype=np.int64)

    # efficiency of the global accesses
    g_w, g_k = np.nonzero(glob)
    gp = pay[g_w, g_k].astype(np.int64)
    gpc = np.minimum((pk[g_w, g_k] & 0xFFFF).astype(np.int64), len(acc) - 1)
    g_eff = np.minimum(1.0, ((((gp >> 16) & 0xFF) * acc[gpc] + 127) // 128) / ((gp >> 8) & 0xFF))
    g_bad = g_eff < RULES["efficiency_critical"]
    uncoalesced = int(((g_eff >= RULES["efficiency_critical"]) & (g_eff < RULES["efficiency_uncoalesced"])).sum())

    # divergence ratio of the divergent branches
    d_w, d_k = np.nonzero(div)
    d_act = words[d_w, d_k, 2]
    d_tak = pay[d_w, d_k] & d_act
    d_ratio = np.minimum(_popc32(d_tak), _popc32(d_act & ~d_tak)) / np.maximum(1, _popc32(d_act))
    d_bad = d_ratio > RULES["divergence_ratio"]

    c_w, c_k = np.nonzero(conflict)
    w_i = np.concatenate([c_w, g_w[g_bad], d_w[d_bad]])
    k_i = np.concatenate([c_k, g_k[g_bad], d_k[d_bad]])
    rule = np.concatenate([np.zeros(len(c_w), np.int64), np.ones(int(g_bad.sum()), np.int64),
                           np.full(int(d_bad.sum()), 2, np.int64)])
    value = np.concatenate([deg[c_w, c_k].astype(np.float64), g_eff[g_bad], d_ratio[d_bad]])
    order = np.lexsort((k_i, w_i))  # warp order, then record order
    w_i, k_i, rule, value = w_i[order], k_i[order], rule[order], value[order]
    return {"warp": w_i, "record": k_i, "pc": (pk[w_i, k_i] & 0xFFFF).astype(np.int64), "rule": rule, "value": value,
            "conflicts": int(len(c_w)), "uncoalesced": uncoalesced, "divergent": int(len(d_w))}


def hints(headers, records, info, occupancy_result=None, warps_per_block=1):
    """Performance hints over extended trace records (one slot per warp), from the
    rule table of hint_table: one hint per record that trips a rule (with its warp,
    block, record index, pc and source line), then the summary and occupancy hints."""
    t = hint_table(headers, records, info)
    lines = [d["line"] for d in info.desc]
    out = []
    for w, k, pc, rule, v in zip(t["warp"].tolist(), t["record"].tolist(), t["pc"].tolist(), t["rule"].tolist(),
                                 t["value"].tolist()):
        where = {"warp": w, "block": w // warps_per_block, "record": k, "pc": pc, "source_line": lines[pc]}
        if rule == 0:
            d = int(v)
            if d >= RULES["degree_critical"]:
                out.append(dict(category="memory", severity="critical", message="shared bank-conflict degree %d" % d,
                                detail="at least %d lanes wait on one bank: this access runs as %d serial passes"
                                % (RULES["degree_critical"], d), degree=d, **where))
            else:
                out.append(dict(category="memory", severity="warning", message="shared bank-conflict degree %d" % d,
                                detail="lanes share a bank at different addresses: %d passes instead of one" % d,
                                degree=d, **where))
        elif rule == 1:
            out.append(dict(category="memory", severity="critical",
                            message="global access at %d%% coalescing efficiency" % int(v * 100),
                            detail="its bytes are spread over far more 128-byte lines than they fill",
                            efficiency=v, **where))
        else:
            out.append(dict(category="divergence", severity="warning",
                            message="branch splits the warp, %d%% of lanes on the smaller side" % int(v * 100),
                            detail="the two sides of this branch run one after the other", ratio=v, **where))
    if t["conflicts"] > RULES["conflicts_summary"]:
        out.append(dict(category="memory", severity="warning",
                        message="%d shared accesses with bank conflicts" % t["conflicts"],
                        detail="lay shared arrays out (padding, a different index) so that a warp's lanes "
                               "fall in distinct banks"))
    if t["divergent"] > RULES["divergent_summary"]:
        out.append(dict(category="divergence", severity="warning",
                        message="%d branches split their warp" % t["divergent"],
                        detail="keep branch conditions uniform across a warp, or turn short branches into selects"))
    if occupancy_result:
        occ, lim = occupancy_result["occupancy_percent"], occupancy_result["limiting_factor"]
        lim = lim.replace("_", " ")
        if occ < RULES["occupancy_critical"]:
            out.append(dict(category="occupancy", severity="critical", message="occupancy %g%%, under a quarter" % occ,
                            detail="%s bound the resident warps; ask for less of them per thread or per block"
                                   % lim))
        elif occ < RULES["occupancy_warning"]:
            out.append(dict(category="occupancy", severity="warning", message="occupancy %g%%, under half" % occ,
                            detail="%s bound the resident warps" % lim))
    return out


def _slot_bytes(headers, records, trace_format):
    """Headers and records back in the slot layout of ks_read_trace (one row per warp)."""
    n_w = len(headers)
    h = np.ascontiguousarray(headers).view(np.uint8).reshape(n_w, 16)
    r = np.ascontiguousarray(records).view(np.uint8).reshape(n_w, -1)
    raw = np.empty((n_w, 16 + r.shape[1]), dtype=np.uint8)
    raw[:, :16] = h
    raw[:, 16:] = r
    return raw


def write_chrome_trace(path, headers, records, info, warps_per_block, trace_format=ks.KS_TRACE_EXTENDED,
                       first_warp=0):
    """Write the per-warp slots as a trace-event JSON file (Chrome / Perfetto): one
    process per block, one thread per warp, one complete event per issued instruction
    from its issue cycle to the warp's next issue (1 cycle for the last); time unit
    one simulated cycle.  The libkscope writer does the formatting; this side only
    supplies each pc's name and source line.  Returns the number of instruction events."""
    names = [json.dumps(info.mnemonic(pc)) for pc in range(len(info.desc))]
    args = ['"pc":%d,"line":%d,"text":%s' % (pc, d["line"], json.dumps(info.text(pc))) for pc, d in enumerate(info.desc)]
    raw = _slot_bytes(headers, records, trace_format)
    return ks.ks_write_trace_events(raw, len(headers), raw.shape[1], trace_format, first_warp, warps_per_block,
                                    names, args, path)


def chrome_trace(headers, records, info, warps_per_block, trace_format=ks.KS_TRACE_EXTENDED, first_warp=0):
    """The document write_chrome_trace writes, parsed into a dict (for small traces)."""
    import os
    import tempfile
    fd, path = tempfile.mkstemp(suffix=".json")
    os.close(fd)
    try:
        write_chrome_trace(path, headers, records, info, warps_per_block, trace_format, first_warp)
        with open(path) as f:
            return json.load(f)
    finally:
        os.unlink(path)


def param_block(ptx, values, entry=None):
    """The parameter block of the program's entry holding `values` (a dict from
    parameter name to an int, or a float for a 4-byte parameter stored as binary32);
    a pointer parameter's value is a byte offset into simulated memory, and a
    parameter not named is 0.  The layout is the library's own (ks_param_info, in
    declaration order at natural alignment), so it is what ks_run reads.  An unknown
    name or a value that does not fit its parameter is a ValueError."""
    import struct
    prog = ks.ks_load_program(ptx, entry)
    try:
        info = ks.ks_program_info(prog)
        buf = bytearray(info["param_bytes"])
        names = set()
        for i in range(info["n_params"]):
            off, size, name = ks.ks_param_info(prog, i)
            names.add(name)
            v = values.get(name, 0)
            if isinstance(v, float):
                if size != 4:
                    raise ValueError("parameter %s has %d bytes: a float needs 4" % (name, size))
                try:
                    raw = struct.pack("<f", v)
                except OverflowError:
                    raise ValueError("value %r of parameter %s is beyond binary32" % (v, name)) from None
            else:
                v = int(v)
                if not -(1 << (8 * size - 1)) <= v < (1 << (8 * size)):
                    raise ValueError("value %d does not fit the %d-byte parameter %s" % (v, size, name))
                raw = (v & ((1 << (8 * size)) - 1)).to_bytes(size, "little")
            buf[off:off + size] = raw
        unknown = sorted(set(values) - names)
        if unknown:
            raise ValueError("no parameter named %s (the entry has %s)" % (", ".join(unknown), ", ".join(sorted(names))))
        return bytes(buf)
    finally:
        ks.ks_program_free(prog)


def _dims(text):
    try:
        d = [int(x) for x in text.split(",")]
    except ValueError:
        raise SystemExit("a grid or block is 1 to 3 comma-separated integers: %s" % text) from None
    if not 1 <= len(d) <= 3:
        raise SystemExit("a grid or block is 1 to 3 comma-separated sizes: %s" % text)
    return tuple(d + [1] * (3 - len(d)))


def main(argv=None):
    """Run a workload on the GPU with extended records and report occupancy, hints
    and (with --out) a Chrome/Perfetto trace of its first warps.  The workload is a
    built-in one, or a PTX file with its launch shape, parameters and initial
    simulated memory (--ptx, --grid, --block, --param, --gmem, --gmem-bytes)."""
    import argparse
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import configs as W
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="vector_add",
                    help="vector_add | strided_<s> | bank_<s> | ffma_<acc> | random_<seed>")
    ap.add_argument("--ptx", default=None, help="simulate this PTX file instead of a built-in workload")
    ap.add_argument("--entry", default=None, help="the .entry to simulate (default: the first)")
    ap.add_argument("--grid", default="1", help="grid size x[,y[,z]] (with --ptx)")
    ap.add_argument("--block", default="32", help="block size x[,y[,z]] (with --ptx)")
    ap.add_argument("--param", action="append", default=[],
                    help="name=value, repeatable (with --ptx); a pointer is a byte offset into simulated memory; "
                         "a value that is not an integer (0x.. allowed) is read as a float")
    ap.add_argument("--gmem", default=None, help="initial simulated memory: a raw byte file (with --ptx)")
    ap.add_argument("--gmem-bytes", type=int, default=None,
                    help="simulated memory size (with --ptx; default the --gmem file's size, else 1 MiB)")
    ap.add_argument("--trace-cap", type=int, default=1024, help="records per warp (with --ptx)")
    ap.add_argument("--arch", default="sm_80")
    ap.add_argument("--out", default=None, help="write the trace-event JSON here")
    ap.add_argument("--dump-gmem", default=None, help="write the simulated memory after the run here (raw bytes)")
    ap.add_argument("--warps", type=int, default=64, help="warps exported to the timeline")
    args = ap.parse_args(argv)
    name = args.workload
    if args.ptx:
        ptx = open(args.ptx).read()
        values = {}
        for kv in args.param:
            k, sep, v = kv.partition("=")
            if not sep:
                raise SystemExit("--param takes name=value: %s" % kv)
            try:
                values[k.strip()] = int(v, 0)
            except ValueError:
                try:
                    values[k.strip()] = float(v)
                except ValueError:
                    raise SystemExit("--param %s: %r is neither an integer nor a float" % (k, v))
        image = np.fromfile(args.gmem, np.uint8) if args.gmem else np.zeros(0, np.uint8)
        size = args.gmem_bytes or (image.size if image.size else 1 << 20)
        if image.size > size:
            raise SystemExit("the --gmem file holds %d bytes, more than --gmem-bytes %d" % (image.size, size))
        gmem = np.zeros(size, np.uint8)
        gmem[:image.size] = image
        grid, block = _dims(args.grid), _dims(args.block)
        w = W.Workload(name=os.path.basename(args.ptx), ptx=ptx, grid=grid, block=block, params=[], gmem=gmem,
                       trace_cap=args.trace_cap)
        pbytes = param_block(ptx, values, args.entry)
    elif name == "vector_add":
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
    if not args.ptx:
        pbytes = w.params_bytes
    s = ks.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=w.trace_cap, trace_format=ks.KS_TRACE_EXTENDED,
                   entry=args.entry)
    try:
        s.load_gmem(w.gmem)
        s.run(pbytes)
        hdr, rec = s.trace_records()
        kernel = s.kernel_name()
        cnt = s.read_counters()
        if args.dump_gmem:
            s.read_gmem().tofile(args.dump_gmem)
    finally:
        s.close()
    info = ProgramInfo(w.ptx, args.entry)
    occ = program_occupancy(w.ptx, w.threads_per_block, args.arch, args.entry)
    hs = hints(hdr, rec, info, occ, w.warps_per_block)
    totals = {f: int(cnt[f].sum()) for f in ("thread_instrs", "warp_instrs", "gld_n", "gld_sectors", "gld_lines",
                                               "gst_n", "gst_sectors", "gst_lines", "sh_n", "sh_degree_sum",
                                               "diverge_n", "barrier_n", "fault_n")}
    totals.update({"warps": int(len(cnt)), "max_cycles": int(cnt["cycles"].max()) if len(cnt) else 0,
                   "max_stack_depth": int(cnt["max_stack_depth"].max()) if len(cnt) else 0,
                   "status_or": int(np.bitwise_or.reduce(cnt["status"])) if len(cnt) else 0})
    print(json.dumps({"workload": w.name, "kernel": kernel, "occupancy": occ, "counters": totals,
                      "hints": [h for h in hs if "warp" not in h] + [h for h in hs if "warp" in h][:20],
                      "n_event_hints": sum(1 for h in hs if "warp" in h)}, indent=1))
    if args.out:
        write_chrome_trace(args.out, hdr[: args.warps], rec[: args.warps], info, w.warps_per_block)


if __name__ == "__main__":
    main()
