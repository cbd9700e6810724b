"""Compile the C oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, FP contraction off, no fast-math, so every FP32 operation in the
oracle is one IEEE round-to-nearest-even step.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
         "-fopenmp", "-Wall", "-Wno-unknown-pragmas"]


def build(force: bool = True) -> str:
    """Compile the oracle; with force=False only when the library is missing or stale."""
    if (not force and os.path.exists(LIB)
            and os.path.getmtime(LIB) >= os.path.getmtime(SRC)):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", *FLAGS, SRC, "-o", tmp, "-lm"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
