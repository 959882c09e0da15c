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
SOURCES = [os.path.join(CSRC, "ks_host.cpp"), os.path.join(CSRC, "ks_kernel.hip"), os.path.join(CSRC, "ks_scratch.hip"),
           os.path.join(CSRC, "ks_clear.hip")]
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
RESERVED_VGPR_KERNELS = ("ks_interp_v32", "ks_interp_v64", "ks_interp_v32_ext", "ks_interp_v64_ext",
                         "ks_interp_v32_cache", "ks_interp_v64_cache")
INTERP_KERNELS = RESERVED_VGPR_KERNELS
# first VGPR of each kernel's register file (compiler-allocated code stays below it)
RESERVED_BASE = {"ks_interp_v32": 56, "ks_interp_v64": 56, "ks_interp_v32_ext": 64, "ks_interp_v64_ext": 64,
                 "ks_interp_v32_cache": 56, "ks_interp_v64_cache": 56}
# register-file VGPRs from RESERVED_BASE on
RF_VGPRS = {"ks_interp_v32": 40, "ks_interp_v64": 72, "ks_interp_v32_ext": 40, "ks_interp_v64_ext": 72,
            "ks_interp_v32_cache": 40, "ks_interp_v64_cache": 72}



class _Flow:
    """Control flow of one kernel body for the index-mode checks.

    Branches are followed both ways except where the compiler steers control flow
    with a flag pair it has just set to a constant: `s_mov_b64 s[a:b], 0` or `-1`,
    then `s_and_b64 vcc, exec, s[a:b]` (vcc = 0 when the pair is 0) or
    `s_andn2_b64 vcc, exec, s[a:b]` (vcc = 0 when it is -1); a vcc known to be 0
    decides the next s_cbranch_vccz / s_cbranch_vccnz.  A pair's constant is
    forgotten at any instruction whose destination names one of its registers.
    A state is (consts, vcc0)."""
    PAIR = re.compile(r"s\[(\d+):(\d+)\]")
    START = (frozenset(), False)

    def __init__(self, body: str):
        self.insts = []
        for line in body.split("\n"):
            t = line.split(";")[0].strip()
            if t and not (t.startswith(".") and not t.endswith(":")):
                self.insts.append(t)
        self.labels = {t[:-1]: i for i, t in enumerate(self.insts) if t.endswith(":")}
        self.n = len(self.insts)

    def op(self, i):
        t = self.insts[i]
        return None if t.endswith(":") else t.split()[0]

    def _dest_regs(self, t):
        """Scalar registers named by an instruction's first operand."""
        parts = t.split(None, 1)
        if len(parts) < 2:
            return set()
        first = parts[1].split(",")[0].strip()
        m = self.PAIR.fullmatch(first)
        if m:
            return set(range(int(m.group(1)), int(m.group(2)) + 1))
        m = re.fullmatch(r"s(\d+)", first)
        if m:
            return {int(m.group(1))}
        if first in ("vcc", "vcc_lo", "vcc_hi"):
            return {"vcc"}
        return set()

    def step(self, i, st):
        """Successors [(index, state)] of instruction i entered in state st."""
        consts, vcc0 = st
        t = self.insts[i]
        n = self.n
        if t.endswith(":"):
            return [(i + 1, st)] if i + 1 < n else []
        parts = t.split()
        op = parts[0]
        d = self._dest_regs(t)
        new_vcc0 = vcc0 and "vcc" not in d and not op.startswith("v_cmp")
        if op in ("s_and_b64", "s_andn2_b64") and t.split(None, 1)[1].replace(" ", "").startswith("vcc,exec,"):
            m = self.PAIR.search(t.split("exec,", 1)[1])
            val = dict(consts).get((int(m.group(1)), int(m.group(2)))) if m else None
            new_vcc0 = (op == "s_and_b64" and val == 0) or (op == "s_andn2_b64" and val == -1)
        if d:
            consts = frozenset(c for c in consts if not (set(range(c[0][0], c[0][1] + 1)) & d))
        if op == "s_mov_b64":
            m = self.PAIR.fullmatch(t.split(None, 1)[1].split(",")[0].strip())
            src = t.split(",", 1)[1].strip()
            if m and src in ("0", "-1"):
                consts = consts | {((int(m.group(1)), int(m.group(2))), int(src))}
        out = (consts, new_vcc0)
        if op == "s_branch":
            return [(self.labels[parts[1]], out)]
        if op.startswith("s_cbranch"):
            tgt = self.labels[parts[1]]
            if op == "s_cbranch_vccz" and vcc0:
                return [(tgt, out)]
            if op == "s_cbranch_vccnz" and vcc0:
                return [(i + 1, out)]
            return [(tgt, out), (i + 1, out)]
        if op in ("s_endpgm", "s_setpc_b64"):
            return []
        return [(i + 1, out)] if i + 1 < n else []


def index_mode_hazards(body: str) -> list:
    """Places in a kernel body where VGPR index mode is switched on while a load
    that returns into a VGPR (vector memory, scratch or LDS) may still be
    outstanding.

    On gfx950 such a load's data was observed to land in the wrong register when
    instructions in index mode ran before it returned.  The check is a forward
    data flow over the body's branches (_Flow): a load sets an outstanding bit
    (vector memory or LDS), `s_waitcnt vmcnt(0)` / `lgkmcnt(0)` clears it, and
    every `s_set_gpr_idx_on` reached with a bit set is reported as (index, text)."""
    f = _Flow(body)
    seen = [set() for _ in range(f.n)]
    work = [(0, 0, f.START)]
    found = {}
    while work:
        i, bits, st = work.pop()
        if i >= f.n or (bits, st) in seen[i]:
            continue
        seen[i].add((bits, st))
        t, op = f.insts[i], f.op(i)
        if op == "s_set_gpr_idx_on" and bits:
            found[i] = t
        if op is not None:
            if re.match(r"(global|buffer|flat|scratch)_load", op) or (re.match(r"(global|buffer|flat)_atomic", op) and " glc" in t):
                bits |= 1
            if re.match(r"ds_(read|load|bpermute|permute|swizzle)", op) or (op.startswith("ds_") and "_rtn" in op):
                bits |= 2
            if op == "s_waitcnt":
                if "vmcnt(0)" in t:
                    bits &= ~1
                if "lgkmcnt(0)" in t:
                    bits &= ~2
        work.extend((j, bits, s2) for j, s2 in f.step(i, st))
    return sorted(found.items())


# Fewest instructions that must separate a vector-memory store from the next
# `s_set_gpr_idx_on` (unless `s_waitcnt vmcnt(0)` comes between them).
STORE_INDEX_GAP = 32


def store_index_gaps(body: str) -> list:
    """For every vector-memory store of a kernel body: (gap, index, text), gap being
    the fewest instructions on any path (_Flow) from the store to an
    `s_set_gpr_idx_on` that no `s_waitcnt vmcnt(0)` separates from it (None: no
    such path).

    On gfx950 an extended-trace record store followed within a handful of
    instructions by index-mode register accesses faulted with an address outside
    every aperture under a full-chip load, while stores 48 or more instructions
    ahead of index mode ran clean at the same load: a store still reading its
    address or data registers when index mode turns on is taken to read them
    through the index."""
    import heapq
    f = _Flow(body)
    out = []
    for i in range(f.n):
        op = f.op(i)
        if op is None or not re.match(r"(global|buffer|flat)_store", op):
            continue
        best = {}
        heap = [(0, j, s2) for j, s2 in f.step(i, f.START)]
        gap = None
        while heap:
            d, j, st = heapq.heappop(heap)
            if j >= f.n or best.get((j, st), 1 << 30) <= d:
                continue
            best[(j, st)] = d
            oj = f.op(j)
            if oj is not None:
                if oj == "s_waitcnt" and "vmcnt(0)" in f.insts[j]:
                    continue
                d += 1
                if oj == "s_set_gpr_idx_on":
                    gap = d - 1
                    break
            for k, s2 in f.step(j, st):
                heapq.heappush(heap, (d, k, s2))
        out.append((gap, i, f.insts[i]))
    return out


def check_device_asm(asm_text: str) -> dict:
    """Check the interpreter kernels' gfx950 assembly; returns per-kernel resources.

    Raises RuntimeError when a kernel spills to scratch, when compiler-written
    code (outside inline asm) in a register-file kernel names a VGPR at or above
    RESERVED_BASE, when such a kernel's VGPR count does not cover its file, or
    when VGPR index mode can be switched on while a load is outstanding
    (index_mode_hazards) or soon after a store (store_index_gaps)."""
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
            base = RESERVED_BASE[k]
            need = base + RF_VGPRS[k]
            if info[k]["vgprs"] < need:
                raise RuntimeError("%s: VGPR count %d does not cover the register file (v%d..v%d)"
                                   % (k, info[k]["vgprs"], base, need - 1))
            if hi >= base:
                raise RuntimeError("%s: compiler-allocated code uses v%d (v%d+ hold the register file)"
                                   % (k, hi, base))
            hz = index_mode_hazards(body)
            if hz:
                raise RuntimeError("%s: VGPR index mode switched on while a load may be outstanding: %s"
                                   % (k, hz[:3]))
            near = [g for g in store_index_gaps(body) if g[0] is not None and g[0] < STORE_INDEX_GAP]
            if near:
                raise RuntimeError("%s: vector-memory store within %d instructions of VGPR index mode: %s"
                                   % (k, STORE_INDEX_GAP, near[:3]))
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
