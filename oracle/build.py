"""Build the fp64 CPU oracle (test infrastructure) with the host C compiler.

    python oracle/build.py

Produces oracle/libkda_oracle.so.  Plain -O2 without fast-math so that the
arithmetic keeps IEEE double semantics; no -march so the library runs on any
x86-64 host.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, SRC,
           "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
