"""Build the CPU oracle shared library (test infrastructure only).

    python oracle/build.py

Compiles ``moe_oracle.c`` with gcc into ``oracle/liboracle.so``.  Strict IEEE
flags: no fast-math, no FMA contraction (every fused multiply-add in the
oracle is an explicit ``fmaf``), OpenMP over tokens and rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

FLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
         "-mfma", "-shared", "-fPIC", "-Wall", "-Wno-unknown-pragmas"]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["gcc", *FLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
