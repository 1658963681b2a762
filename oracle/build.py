"""Build the CPU oracle library (test infrastructure only).

The oracle is plain C, compiled with -ffp-contract=off and without fast-math so
that every binary32 operation is a single IEEE round-to-nearest-even operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
        "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
