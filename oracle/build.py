"""Build the CPU oracle shared library (test infrastructure only).

The oracle is plain C compiled by gcc with IEEE fp32 semantics: no FMA
contraction and no fast-math, so that its fp32 quantisation decisions are
the textbook round-to-nearest-even ones.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_nvfp4.so")
SRC = os.path.join(HERE, "nvfp4_oracle.c")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
