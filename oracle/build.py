"""Compile the FP64 CPU oracle (test infrastructure) into oracle/liboracle_rmsn.so.

Plain gcc, -O2, no fast-math, no FMA contraction: the oracle's double
arithmetic is exactly the sequence of operations written in rmsn_oracle.c.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rmsn_oracle.c")
LIB = os.path.join(HERE, "liboracle_rmsn.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
        "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    # A planted-mistake copy of the oracle (tests/test_oracle_mutations.py)
    # is selected through this variable; nothing else sets it.
    override = os.environ.get("RMSN_ORACLE_LIB")
    if override:
        return override
    if (not os.path.exists(LIB)) or os.path.getmtime(LIB) < max(
        os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "rmsn_oracle.h"))
    ):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
