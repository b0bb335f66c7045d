"""Build the CPU oracle (test infrastructure) with gcc.

The oracle is plain C compiled without fast-math and without FP contraction,
so every double operation is a single IEEE-rounded step.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rmsq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# The same source without OpenMP (its pragmas ignored): one thread by
# construction, for timing the oracle on a single core whatever thread count
# the host's OpenMP runtime imposes.
LIB_SERIAL = os.path.join(HERE, "liboracle_serial.so")


def _compile(out: str, openmp: bool, verbose: bool) -> None:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           *(["-fopenmp"] if openmp else ["-Wno-unknown-pragmas"]),
           "-Wall", "-Wextra", "-shared", "-fPIC", SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    _compile(LIB, True, verbose)
    _compile(LIB_SERIAL, False, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
