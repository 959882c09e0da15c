"""Build libkscope.so (host front end + gfx950 interpreter) in-tree with hipcc.

Flags that matter for results:
  -ffp-contract=off        single-precision add/mul stay separately rounded
                           (fma.rn.f32 is an explicit fused multiply-add)
  no fast-math, no flush   subnormals are kept
  -packed-fp32-ops off     no v_pk_* f32 instructions are generated
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkscope.so")
SOURCES = [os.path.join(CSRC, "ks_host.cpp"), os.path.join(CSRC, "ks_kernel.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-fno-gpu-rdc", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument", "-Wno-inline-asm"]


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in SOURCES + [os.path.join(CSRC, f) for f in os.listdir(CSRC)])
        if os.path.getmtime(LIB) >= newest:
            return LIB
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
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", out_path,
           os.path.join(CSRC, "ks_kernel.hip")]
    subprocess.run(cmd, check=True, cwd=HERE)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
