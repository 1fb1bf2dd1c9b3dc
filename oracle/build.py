"""Build the CPU oracle (test infrastructure): oracle/liblsa_ref.so from oracle/lsa_ref.c.

Plain C11, OpenMP over independent rows, no FMA contraction (the page-key mean is defined with a
fixed binary32 rounding sequence, which contraction would change).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lsa_ref.c")
LIB = os.path.join(HERE, "liblsa_ref.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
