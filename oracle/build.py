"""Compile the C oracle into oracle/liboracle.so with gcc.

Test infrastructure only (see oracle.h).  The flags keep every binary32
operation as written: no contraction into fused multiply-add, no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=gnu99", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fno-builtin-fmaf",
        "-Wall", "-Wextra", "-Werror",
        os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
