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
RESERVED_VGPR_KERNELS = ("ks_interp_v32", "ks_interp_v64", "ks_interp_v32_ext", "ks_interp_v64_ext")
INTERP_KERNELS = RESERVED_VGPR_KERNELS
# first VGPR of each kernel's register file (compiler-allocated code stays below it)
RESERVED_BASE = {"ks_interp_v32": 56, "ks_interp_v64": 56, "ks_interp_v32_ext": 64, "ks_interp_v64_ext": 64}
# register-file VGPRs from RESERVED_BASE on
RF_VGPRS = {"ks_interp_v32": 40, "ks_interp_v64": 72, "ks_interp_v32_ext": 40, "ks_interp_v64_ext": 72}



def index_mode_hazards(body: str) -> list:
    """Places in a kernel body where VGPR index mode is switched on while a load
    that returns into a VGPR (vector memory, scratch or LDS) may still be
    outstanding.

    On gfx950 such a load's data was observed to land in the wrong register when
    instructions in index mode ran before it returned.  The check is a forward
    data flow over the body's branches: a load sets an outstanding bit (vector
    memory or LDS), `s_waitcnt vmcnt(0)` / `lgkmcnt(0)` clears it, and every
    `s_set_gpr_idx_on` reached with a bit set is reported as (index, text).

    Branches are followed both ways except where the compiler steers control flow
    with a flag pair it has just set to a constant: `s_mov_b64 s[a:b], 0` or `-1`,
    then `s_and_b64 vcc, exec, s[a:b]` (vcc = 0 when the pair is 0) or
    `s_andn2_b64 vcc, exec, s[a:b]` (vcc = 0 when it is -1); a vcc known to be 0
    decides the next s_cbranch_vccz / s_cbranch_vccnz.  A pair's constant is
    forgotten at any instruction whose destination names one of its registers."""
    insts = []
    for line in body.split("\n"):
        t = line.split(";")[0].strip()
        if t and not (t.startswith(".") and not t.endswith(":")):
            insts.append(t)
    labels = {t[:-1]: i for i, t in enumerate(insts) if t.endswith(":")}
    n = len(insts)
    pair_re = re.compile(r"s\[(\d+):(\d+)\]")

    def dest_regs(t):
        """Scalar registers named by an instruction's first operand."""
        parts = t.split(None, 1)
        if len(parts) < 2:
            return set()
        first = parts[1].split(",")[0].strip()
        m = pair_re.fullmatch(first)
        if m:
            return set(range(int(m.group(1)), int(m.group(2)) + 1))
        m = re.fullmatch(r"s(\d+)", first)
        if m:
            return {int(m.group(1))}
        if first in ("vcc", "vcc_lo", "vcc_hi"):
            return {"vcc"}
        return set()

    def step(i, st):
        """Successor states of instruction i from state st = (bits, consts, vcc0)."""
        bits, consts, vcc0 = st
        t = insts[i]
        if t.endswith(":"):
            return [(i + 1, st)] if i + 1 < n else []
        parts = t.split()
        op = parts[0]
        if re.match(r"(global|buffer|flat|scratch)_load", op) or (re.match(r"(global|buffer|flat)_atomic", op) and " glc" in t):
            bits |= 1
        if re.match(r"ds_(read|load|bpermute|permute|swizzle)", op) or (op.startswith("ds_") and "_rtn" in op):
            bits |= 2
        if op == "s_waitcnt":
            if "vmcnt(0)" in t:
                bits &= ~1
            if "lgkmcnt(0)" in t:
                bits &= ~2
        d = dest_regs(t)
        new_vcc0 = vcc0 and "vcc" not in d and not op.startswith("v_cmp")
        if op in ("s_and_b64", "s_andn2_b64") and t.split(None, 1)[1].replace(" ", "").startswith("vcc,exec,"):
            m = pair_re.search(t.split("exec,", 1)[1])
            val = dict(consts).get((int(m.group(1)), int(m.group(2)))) if m else None
            new_vcc0 = (op == "s_and_b64" and val == 0) or (op == "s_andn2_b64" and val == -1)
        if d:
            consts = frozenset(c for c in consts if not (set(range(c[0][0], c[0][1] + 1)) & d))
        if op == "s_mov_b64":
            m = pair_re.fullmatch(t.split(None, 1)[1].split(",")[0].strip())
            src = t.split(",", 1)[1].strip()
            if m and src in ("0", "-1"):
                consts = consts | {((int(m.group(1)), int(m.group(2))), int(src))}
        out = (bits, consts, new_vcc0)
        if op == "s_branch":
            return [(labels[parts[1]], out)]
        if op.startswith("s_cbranch"):
            tgt = labels[parts[1]]
            if op == "s_cbranch_vccz" and vcc0:
                return [(tgt, out)]
            if op == "s_cbranch_vccnz" and vcc0:
                return [(i + 1, out)]
            return [(tgt, out), (i + 1, out)]
        if op in ("s_endpgm", "s_setpc_b64"):
            return []
        return [(i + 1, out)] if i + 1 < n else []

    # states per instruction: a set of (bits, consts, vcc0); small in practice
    seen = [set() for _ in range(n)]
    work = [(0, (0, frozenset(), False))]
    found = {}
    while work:
        i, st = work.pop()
        if i >= n or st in seen[i]:
            continue
        seen[i].add(st)
        t = insts[i]
        if not t.endswith(":") and t.split()[0] == "s_set_gpr_idx_on" and st[0]:
            found[i] = t
        work.extend(step(i, st))
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
