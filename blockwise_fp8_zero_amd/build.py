"""Build blockwise_fp8_zero_amd/libbfz.so for gfx950 with hipcc (in-tree)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbfz.so")
SOURCES = ["plan.cpp", "abi.cpp", "kernels.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fno-fast-math",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def build(verbose: bool = False) -> str:
    objs = []
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(obj_dir, src + ".o")
        cmd = ["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
           "-Wl,--version-script=" + os.path.join(CSRC, "exports.map"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
