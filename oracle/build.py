"""Compile the C oracle into ``oracle/libce_oracle.so`` with gcc.

Test infrastructure only (see ``ce_oracle.c``).  Plain ``-O2``: no fast-math
(inf/NaN semantics and log1p matter), no FMA contraction, OpenMP over rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ce_oracle.c")
LIB = os.path.join(HERE, "libce_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
