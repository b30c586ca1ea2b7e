"""Compile the CPU oracle (plain C99, gcc) into oracle/liboracle.so.

Test infrastructure: the oracle is built so the tests, the smoke check and
the benchmark's CPU-baseline leg can call it.  Run as a script or call
``build()``; it always recompiles.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "qmm_oracle.c")
    tmp = LIB + ".tmp"
    # -ffp-contract=off: every product and sum is rounded as written.
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
