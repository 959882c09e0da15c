#!/usr/bin/env python3
"""Benchmark: simulated thread-instructions/s and analysed warp-accesses/s on one GPU.

One step = one ks_run of the whole hot path (fetch/issue/execute, divergence
stack, scoreboard, sector/line/bank analyser, trace and counter writes) over
the random-stress workload: 65536 x 256 = 16.8 M simulated threads running a
seeded 2000-instruction program of the PTX subset over 1 GiB of simulated
global memory, trace cap 2048 records per warp.  Inputs are resident in HBM
before timing starts.

Prints one JSON line (rank 0).  `roofline` prices the interpreter kernel's
algorithmic bytes (32 B per counted sector + 8 B per written trace record +
16 B header and 80 B counters per warp) per launch against MI355X's 8 TB/s HBM;
the launch duration comes from HIP events on the launch stream.
`hbm_measured` prices the rocprofv3 FETCH_SIZE/WRITE_SIZE bytes of the same
kernel (from the committed counter summary, when it was taken on the current
kernel source) the same way.  `launch_ms` gives min, median, mean, max, std, p5
and p95 of the per-launch HIP-event times, whose raw values go to a CSV file; a
plain 1 GiB device copy is timed in the same run as the achievable ceiling.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload
(with every host thread, and on one thread over 1/64 of that sample), and
reports whether its counter records equal the GPU's.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "simulated thread-instr/s + analysed warp-accesses/s at 1 GPU; % HBM peak"


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("ks_kernel.hip", "ks_isa.h"):
        with open(os.path.join(ROOT, "analysis_ptxsimulator_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_counters(workload_key):
    """The committed rocprofv3 counter summary of this workload (HBM bytes per
    launch from FETCH_SIZE/WRITE_SIZE, VALU utilisation), if it was taken on the
    current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload_key)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d


def make_workload(name):
    from workloads import configs as W
    if name == "random_stress":
        return W.random_stress(prog_seed=0)
    if name.startswith("random_stress_g"):  # the same program and memory on fewer blocks
        return W.random_stress(prog_seed=0, grid=int(name[15:]))
    if name == "ffma_dep":
        return W.ffma_probe(n_acc=1)
    if name == "ffma_ind":
        return W.ffma_probe(n_acc=8)
    if name.startswith("bank_s"):
        return W.bank_probe(int(name[6:]))
    if name.startswith("strided_s"):
        return W.strided_gather(int(name[9:]))
    if name == "vector_add":
        return W.vector_add()
    raise SystemExit("unknown workload %s" % name)


def describe(w):
    m = w.meta
    if w.name.startswith("random_stress"):
        return ("random_stress: %d x %d threads (%.3gM), %d-instruction PTX program seed %d, %d MiB simulated "
                "memory seed %d, trace cap %d" % (w.grid[0], w.block[0], w.n_blocks * w.threads_per_block / 1e6,
                                                   m["n_instr"], m["prog_seed"], w.gmem.size >> 20, m["mem_seed"],
                                                   w.trace_cap))
    return "%s: grid %s block %s trace cap %d" % (w.name, w.grid, w.block, w.trace_cap)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, sample_blocks, threads, cache_model=False, gpu_counters=None):
    """The oracle, as it stands, on blocks [0, sample_blocks) with `threads` host
    threads, then on one thread over the first 1/64 of them.  With the GPU's
    counter records of the same run, reports whether the oracle's are identical."""
    from oracle import oracle as O
    import numpy as np

    def timed(nb, nthreads):
        g = w.gmem  # the sampled blocks only write their own thread-private words
        cache = np.zeros(nb * w.warps_per_block * O.CACHE_WARP_BYTES, np.uint8) if cache_model else None
        t0 = time.perf_counter()
        c, _, _ = O.run(w.ptx, w.grid, w.block, w.params_bytes, g, trace_cap=w.trace_cap, blocks=list(range(nb)),
                        threads=nthreads, cache=cache)
        return c, time.perf_counter() - t0

    c, dt = timed(sample_blocks, threads)
    ti = int(c["thread_instrs"].sum())
    out = {"value": ti / dt, "unit": "thread-instr/s", "cores": threads, "kind": "oracle",
           "sample": "%d of %d blocks (%d thread-instructions) of the same workload, %.2f s wall"
                     % (sample_blocks, w.n_blocks, ti, dt),
           "warp_accesses_per_s": int((c["gld_n"].astype(np.uint64) + c["gst_n"] + c["sh_n"]).sum()) / dt,
           "cpu_model": cpu_model()}
    if gpu_counters is not None:
        out["counters_equal_gpu"] = bool(np.array_equal(c, gpu_counters[:len(c)]))
    nb1 = max(1, sample_blocks // 64)
    c1, dt1 = timed(nb1, 1)
    out["single_thread"] = {"value": int(c1["thread_instrs"].sum()) / dt1, "unit": "thread-instr/s",
                            "sample": "%d blocks (1/64 of the sample), %.2f s wall" % (nb1, dt1)}
    return out


def launch_stats(launch_ms):
    import numpy as np
    a = np.asarray(launch_ms, dtype=np.float64)
    return {"min": float(a.min()), "median": float(np.median(a)), "mean": float(a.mean()), "max": float(a.max()),
            "std": float(a.std(ddof=1)) if a.size > 1 else 0.0, "p5": float(np.percentile(a, 5)),
            "p95": float(np.percentile(a, 95)), "n": int(a.size)}


def write_csv(path, launch_ms):
    d = os.path.dirname(path)
    if d:
        os.makedirs(d, exist_ok=True)
    with open(path, "w") as f:
        f.write("launch,ms\n")
        for k, v in enumerate(launch_ms):
            f.write("%d,%.6f\n" % (k, v))


def copy_ceiling(dev, reps=5):
    """GB/s (bytes read + written) of a plain 1 GiB device-to-device copy."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    dt = (time.perf_counter() - t0) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / dt / 1e9


def copy_calibration(args, dev):
    """A plain 1 GiB device-to-device copy: the achievable-bandwidth ceiling and the
    reference kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"workload": "copy", "bytes_read_per_step": n, "bytes_written_per_step": n,
                      "ms_per_step": dt * 1e3, "GBps_read_plus_write": 2 * n / dt / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--csv", default=None,
                    help="raw per-launch times (default $KS_BENCH_OUT/launch_ms_<workload>.csv, KS_BENCH_OUT "
                         "defaulting to bench_out)")
    ap.add_argument("--workload", default="random_stress")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-blocks", type=int, default=65536)
    ap.add_argument("--cache-model", choices=("none", "warp"), default="none",
                    help="ld.global latency: the fixed table (the timed default) or per-warp L1/L2 caches")
    ap.add_argument("--trace-format", choices=("basic", "extended"), default="basic",
                    help="trace records: 8-byte {cycle, pc} (the timed default) or 16-byte with kind, mask and "
                         "payload (launched 32 blocks at a time, e.g. --workload random_stress_g32)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this simulator's hot path is a single-GPU kernel "
              "(blocks never communicate, so a launch would shard by block ranges, one range per GPU). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from analysis_ptxsimulator_amd import ks

    dev = torch.device("cuda:0")
    if args.workload == "copy":
        return copy_calibration(args, dev)
    w = make_workload(args.workload)
    cache_on = args.cache_model == "warp"
    ext = args.trace_format == "extended"
    s = ks.Session(w.ptx, w.grid, w.block, w.gmem.size, trace_cap=w.trace_cap, device=dev,
                   cache_model=ks.KS_CACHE_WARP if cache_on else ks.KS_CACHE_NONE,
                   trace_format=ks.KS_TRACE_EXTENDED if ext else ks.KS_TRACE_BASIC)
    s.load_gmem(w.gmem)
    params = w.params_bytes
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        s.run(params)
    torch.cuda.synchronize(dev)

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for k in range(args.steps):
        starts[k].record(stream)
        s.run(params)
        ends[k].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    ms_per_step = wall * 1000.0 / args.steps

    c = s.read_counters()
    status = s.status()
    kernel = s.kernel_name()
    ch = s.read_cache_headers() if cache_on else None
    s.close()
    thread_instrs = int(c["thread_instrs"].sum())
    warp_acc = int(c["gld_n"].astype(np.uint64).sum() + c["gst_n"].sum() + c["sh_n"].sum())
    sectors = int(c["gld_sectors"].astype(np.uint64).sum() + c["gst_sectors"].sum())
    records = int(np.minimum(c["warp_instrs"], w.trace_cap).astype(np.uint64).sum())
    alg_bytes = 32 * sectors + (16 if ext else 8) * records + (16 + 80) * len(c)
    cache_stats = None
    if cache_on:
        # the cache model's own state: every warp's caches cleared per run, a 4-byte L1
        # tag read per access, on an L1 miss an L1 tag write and an L2 tag read, on an
        # L2 miss an L2 tag write, and the 16-byte header
        l1h, l2h, miss = (int(ch[f].astype(np.uint64).sum()) for f in ("l1_hits", "l2_hits", "misses"))
        alg_bytes += len(c) * ks.KS_CACHE_WARP_BYTES + 4 * (l1h + l2h + miss) + 8 * (l2h + miss) + 4 * miss
        cache_stats = {"l1_hits": l1h, "l2_hits": l2h, "misses": miss,
                       "state_bytes": len(c) * ks.KS_CACHE_WARP_BYTES}
    avg_launch_s = float(np.mean(launch_ms)) / 1000.0
    achieved = alg_bytes / avg_launch_s / 1e9
    prof = measured_counters(args.workload + ("_cache" if cache_on else "") + ("_ext" if ext else ""))
    traffic = prof.get("hbm_bytes_per_launch") if prof else None
    csv_path = args.csv or os.path.join(os.environ.get("KS_BENCH_OUT", "bench_out"), "launch_ms_%s.csv" % args.workload)
    write_csv(csv_path, launch_ms)
    copy_gbs = copy_ceiling(dev)
    valu = None
    if prof and "valu_busy" in prof:
        valu = {"busy": prof["valu_busy"], "lane_util": prof["valu_lane_util"], "salu_busy": prof["salu_busy"],
                "source": "rocprofv3 counters, profiles/traffic_%s.json" % args.workload}

    out = {
        "metric": METRIC,
        "value": thread_instrs / (ms_per_step / 1000.0),
        "unit": "thread-instr/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": describe(w), "threads": w.n_blocks * w.threads_per_block,
                   "warps": len(c), "parallelism": "single GPU",
                   "ld_global_latency": "per-warp L1/L2 cache model" if cache_on else "fixed table",
                   "trace_format": args.trace_format},
        "warp_accesses_per_s": warp_acc / (ms_per_step / 1000.0),
        "thread_instrs_per_step": thread_instrs,
        "warp_accesses_per_step": warp_acc,
        "run_status_bits": status,
        "launch_ms": dict(launch_stats(launch_ms), csv=csv_path),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": alg_bytes,
                     "kernel": kernel},
        # HBM bandwidth as rocprofv3 measures it: FETCH_SIZE x 2 + WRITE_SIZE bytes (each
        # scaled by a plain copy) per launch over the mean launch time; null when the
        # committed counters were taken on another kernel source
        "hbm_measured": ({"GBps": traffic / avg_launch_s / 1e9, "frac": traffic / avg_launch_s / 1e9 / HBM_PEAK_GBS,
                          "bytes_per_launch": traffic,
                          "source": "rocprofv3 FETCH_SIZE/WRITE_SIZE, profiles/traffic_%s.json" % args.workload}
                         if traffic else None),
        "copy_ceiling_GBps": copy_gbs,
        "valu_utilisation": valu,
    }
    if cache_on:
        out["cache_model"] = cache_stats
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        # the cache model's oracle holds 200 KB of state per warp: a smaller sample
        sample = min(args.cpu_sample_blocks, w.n_blocks, 1024 if cache_on else w.n_blocks)
        out["cpu_baseline"] = cpu_baseline(w, sample, threads, cache_on, gpu_counters=c)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
