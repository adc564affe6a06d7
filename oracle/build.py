"""Compile the oracle's C source into ``oracle/libkda_oracle.so`` with gcc.

Test infrastructure: only the test suite, the smoke check and the benchmark's
CPU-baseline leg load the result.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "kda_oracle.c")
    tmp = LIB + ".tmp"
    # -O2 without -ffast-math: IEEE fp64, no FMA contraction on x86-64 baseline.
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
