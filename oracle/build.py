"""Build the CPU oracle library (test infrastructure only).

The oracle is compiled with the host compiler, contraction of multiply-adds off
and no fast-math, so that its single-precision results are IEEE-754 round to
nearest even, bit for bit.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libks_oracle.so")
SRC = os.path.join(HERE, "ks_oracle.cpp")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-pthread", "-o", tmp, SRC]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
