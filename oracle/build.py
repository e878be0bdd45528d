"""Build the CPU oracle (plain C, gcc) into oracle/libnvfp4_oracle.so.

Test infrastructure: the oracle is built next to the product but never linked
into it.  Flags keep IEEE fp32 semantics: no fast-math, no FMA contraction.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
