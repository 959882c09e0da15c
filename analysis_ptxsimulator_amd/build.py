"""Build libkscope.so (host front end + gfx950 interpreter) in-tree with hipcc.

Flags that matter for results:
  -ffp-contract=off        no multiply-add contraction beyond the explicit fmaf
  no fast-math, no flush   subnormals are kept
  -packed-fp32-ops off     no v_pk_* f32 instructions are generated
"""
import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkscope.so")
SOURCES = [os.path.join(CSRC, "ks_host.cpp"), os.path.join(CSRC, "ks_kernel.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Uniform branches (all of the interpreter's dispatch) need no structurizing: the
# hardware takes them as scalar branches.  Leaving those regions alone removes the
# flow-mask bookkeeping the structurizer would add to every step.
CODEGEN = ["-mllvm", "-structurizecfg-skip-uniform-regions=true"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-fno-gpu-rdc", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument", "-Wno-inline-asm"] + CODEGEN


# The VGPR register-file kernels keep simulated registers in v56 and up, which
# the compiler must never allocate (they are reserved by amdgpu_num_vgpr), and
# their VGPR count must cover the file; no interpreter may use scratch memory.
RESERVED_VGPR_KERNELS = ("ks_interp_v32", "ks_interp_v64")
INTERP_KERNELS = RESERVED_VGPR_KERNELS
RESERVED_BASE = 56
RF_VGPRS = {"ks_interp_v32": 40, "ks_interp_v64": 72}  # register-file VGPRs from RESERVED_BASE on


def index_mode_hazards(body: str) -> list:
    """Places in a kernel body where VGPR index mode is switched on while a load
    that returns into a VGPR (vector memory or LDS) may still be outstanding.

    On gfx950 such a load's data was observed to land in the wrong register when
    instructions in index mode ran before it returned.  The check is a forward
    data flow over the body's branches: a load sets an outstanding bit (vector
    memory or LDS), `s_waitcnt vmcnt(0)` / `lgkmcnt(0)` clears it, and every
    `s_set_gpr_idx_on` reached with a bit set is reported as (index, text).  It
    follows every branch edge, so it may report paths that correlated branch
    conditions never take; the kernels are written so that it reports none."""
    insts = []
    for line in body.split("\n"):
        t = line.split(";")[0].strip()
        if t and not (t.startswith(".") and not t.endswith(":")):
            insts.append(t)
    labels = {t[:-1]: i for i, t in enumerate(insts) if t.endswith(":")}
    n = len(insts)

    def successors(i):
        parts = insts[i].split()
        op = parts[0]
        if op == "s_branch":
            return [labels[parts[1]]]
        if op.startswith("s_cbranch"):
            return [labels[parts[1]], i + 1]
        if op in ("s_endpgm", "s_setpc_b64"):
            return []
        return [i + 1] if i + 1 < n else []

    seen = [0] * n
    visited = [False] * n
    work = [(0, 0)]
    found = {}
    while work:
        i, st = work.pop()
        if i >= n or (visited[i] and (seen[i] | st) == seen[i]):
            continue
        visited[i] = True
        seen[i] |= st
        st = seen[i]
        t = insts[i]
        op = "" if t.endswith(":") else t.split()[0]
        out = st
        if re.match(r"(global|buffer|flat|scratch)_load", op) or (re.match(r"(global|buffer|flat)_atomic", op) and " glc" in t):
            out |= 1
        if re.match(r"ds_(read|load|bpermute|permute|swizzle)", op) or (op.startswith("ds_") and "_rtn" in op):
            out |= 2
        if op == "s_waitcnt":
            if "vmcnt(0)" in t:
                out &= ~1
            if "lgkmcnt(0)" in t:
                out &= ~2
        if op == "s_set_gpr_idx_on" and st:
            found[i] = t
        for j in successors(i):
            work.append((j, out))
    return sorted(found.items())


def check_device_asm(asm_text: str) -> dict:
    """Check the interpreter kernels' gfx950 assembly; returns per-kernel resources.

    Raises RuntimeError when a kernel spills to scratch, when compiler-written
    code (outside inline asm) in a register-file kernel names a VGPR at or above
    RESERVED_BASE, when such a kernel's VGPR count does not cover its file, or
    when VGPR index mode can be switched on while a load is outstanding
    (index_mode_hazards)."""
    info = {}
    for k in INTERP_KERNELS:
        m = re.search(r"^(_Z\d+%sN2ks6KsArgsE):[^\n]*\n(.*?)^\.Lfunc_end" % k, asm_text, re.S | re.M)
        if not m:
            raise RuntimeError("kernel %s not found in device assembly" % k)
        body = m.group(2)
        meta = re.search(r"\.name:\s+%s\n" % re.escape(m.group(1)), asm_text)
        md = asm_text[meta.start():meta.start() + 4000] if meta else ""
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", md)
        vg = re.search(r"\.vgpr_count:\s+(\d+)", md)
        sg = re.search(r"\.sgpr_count:\s+(\d+)", md)
        info[k] = {"scratch": int(priv.group(1)) if priv else -1, "vgprs": int(vg.group(1)) if vg else -1,
                   "sgprs": int(sg.group(1)) if sg else -1}
        if info[k]["scratch"] != 0:
            raise RuntimeError("%s uses %s bytes of scratch" % (k, info[k]["scratch"]))
        if k in RESERVED_VGPR_KERNELS:
            outside, inside = [], False
            for line in body.split("\n"):
                if ";;#ASMSTART" in line:
                    inside = True
                elif ";;#ASMEND" in line:
                    inside = False
                elif not inside:
                    outside.append(line.split(";")[0])
            hi = 0
            for line in outside:
                # VGPR operands: vN or a range v[N:M]
                for lo, top, single in re.findall(r"\bv(?:\[(\d+):(\d+)\]|(\d+)\b)", line):
                    hi = max(hi, int(top or single))
            info[k]["max_compiler_vgpr"] = hi
            need = RESERVED_BASE + RF_VGPRS[k]
            if info[k]["vgprs"] < need:
                raise RuntimeError("%s: VGPR count %d does not cover the register file (v%d..v%d)"
                                   % (k, info[k]["vgprs"], RESERVED_BASE, need - 1))
            if hi >= RESERVED_BASE:
                raise RuntimeError("%s: compiler-allocated code uses v%d (v%d+ hold the register file)"
                                   % (k, hi, RESERVED_BASE))
            hz = index_mode_hazards(body)
            if hz:
                raise RuntimeError("%s: VGPR index mode switched on while a load may be outstanding: %s"
                                   % (k, hz[:3]))
    return info


def build(force: bool = True, verbose: bool = False, check: bool = True) -> str:
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in SOURCES + [os.path.join(CSRC, f) for f in os.listdir(CSRC)])
        if os.path.getmtime(LIB) >= newest:
            return LIB
    if check:
        with tempfile.TemporaryDirectory() as td:
            info = check_device_asm(open(device_asm(os.path.join(td, "k.s"))).read())
        if verbose:
            print(info, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_path: str) -> str:
    """Write the gfx950 assembly of the interpreter (for inspection)."""
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-inline-asm"] + CODEGEN + ["-o", out_path,
           os.path.join(CSRC, "ks_kernel.hip")]
    subprocess.run(cmd, check=True, cwd=HERE)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
