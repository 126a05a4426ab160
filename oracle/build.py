"""Builds the fp64 oracle (test infrastructure) with the host C compiler.

Plain ``-O2``: no ``-ffast-math`` and no contraction of a*b+c into fused
multiply-adds beyond what ISO C allows, so the oracle's arithmetic is the
written one.
"""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mla_oracle.c")
LIB = os.path.join(HERE, "liboracle_mla.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", lib + ".tmp", src, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
