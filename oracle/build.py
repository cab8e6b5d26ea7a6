"""Build the fp64 CPU oracle (plain C, gcc, OpenMP) into oracle/liboracle.so.

Test infrastructure only: the library built here is loaded by the tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["sdm_oracle.c", "gdn_oracle.c", "sse_oracle.c"]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile every oracle source with gcc -O2 -fopenmp (no fast-math) and return the path."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB + ".tmp"] + [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
