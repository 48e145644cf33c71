"""Build synth/libsynth.so (host + gfx950 device code) with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsynth.so")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    cmd = ["hipcc", *HIP_FLAGS, os.path.join(HERE, "synth.hip"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
