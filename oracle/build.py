"""Build the fp64 CPU oracle (liboracle.so) with gcc -- TEST INFRASTRUCTURE.

Building the checker is part of the package build; running it is reserved to
the tests, the smoke check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # -ffp-contract=off: keep every multiply and add a separate fp64 rounding,
    # as written in the source. No -march: the library travels to other hosts.
    cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
