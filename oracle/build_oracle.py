"""Compiles the C twin of the oracle into ``oracle/liboracle_cpu.so`` (gcc, OpenMP).

Test infrastructure: the library is loaded only by the tests, the smoke check
and the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_cpu.c")
LIB = os.path.join(HERE, "liboracle_cpu.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
