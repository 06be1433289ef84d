"""Build the FP64 CPU oracle (test infrastructure) with gcc.

Compiles ``oracle.c`` into ``liboracle.so`` beside it.  Plain C99 + POSIX
threads; no fast-math and no floating-point contraction, so every sum is the
sequential one the source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=gnu99", "-O2", "-fPIC", "-shared", "-pthread",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
