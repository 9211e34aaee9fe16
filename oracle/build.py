"""Build the CPU oracle shared library (plain C, gcc, single-threaded).

TEST INFRASTRUCTURE ONLY: the product library never builds, loads or calls it.
Flags keep every binary32 operation rounded on its own: no contraction into
FMA, no fast-math, SSE arithmetic on x86-64 (FLT_EVAL_METHOD == 0).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-builtin-fmaf", "-Wall", "-Wextra", "-Werror"]


def build(force=True):
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
