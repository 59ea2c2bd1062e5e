"""Build the fp64 CPU oracle (TEST INFRASTRUCTURE) into oracle/libkda_oracle.so.

Plain gcc, -O2, OpenMP, no fast-math: the oracle must keep IEEE semantics
(exp(-inf) = 0, no reassociation).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    """Build if the library is missing or older than its source."""
    if (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
