"""Compile the CPU oracle (plain C, double precision) into ``liboracle_sru.so``.

Test infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline leg load the result; the product path never does.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sru_oracle.c")
LIB = os.path.join(HERE, "liboracle_sru.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
