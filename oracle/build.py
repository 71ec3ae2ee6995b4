"""Compile the CPU oracle (``emb_oracle.c``) into ``oracle/libemb_oracle.so`` with gcc.

Test infrastructure only: the library built here is loaded by the test suite, the smoke
check and the benchmark's CPU-baseline leg, never by the product path.

The flags keep the arithmetic plain: ``-ffp-contract=off`` (no fused multiply-add, every
product and sum is rounded on its own) and no fast-math, so ``nearbyint`` keeps the IEEE
round-to-nearest-even mode.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "emb_oracle.c")
LIB = os.path.join(HERE, "libemb_oracle.so")
# The same source built with OpenMP (the independent bags / samples of the forward and the
# interaction backward over all host threads); only the CPU-baseline timing uses it, and a
# CPU test checks that it gives the plain build's bits.
LIB_OMP = os.path.join(HERE, "libemb_oracle_omp.so")


def build(verbose: bool = False) -> str:
    base = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
            "-Wall", "-Wextra"]
    for lib, extra in ((LIB, ["-Wno-unknown-pragmas"]), (LIB_OMP, ["-fopenmp"])):
        cmd = base + extra + ["-o", lib + ".tmp", SRC, "-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
