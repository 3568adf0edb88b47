"""Compile the fp64 CPU oracle (plain C + OpenMP) into oracle/libe3oracle.so.

Test infrastructure: the oracle is built next to the product so that the
test suite, the smoke check and the benchmark's CPU-baseline leg can load it.
Nothing in the product package imports this module.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "e3_oracle.c")
LIB = os.path.join(HERE, "libe3oracle.so")


def build_oracle(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
