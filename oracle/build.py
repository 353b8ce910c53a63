"""Compile the CPU oracle (``mx_ref.c``) into ``oracle/libmxref.so`` with gcc.

Test infrastructure only.  The flags keep every fp32 expression a single IEEE
operation: no FMA contraction, no fast-math, SSE arithmetic (x86-64 default).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mx_ref.c")
LIB = os.path.join(HERE, "libmxref.so")

FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
         "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
         "-Wall", "-Wno-unknown-pragmas"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *FLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
