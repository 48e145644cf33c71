"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two throw-away builds with gcc / g++ (no GPU code in either):
* the C oracle with tests/sanitize/oracle_driver.c, which drives every
  oracle entry point on exact-size buffers;
* the library's planner and C ABI (plan.cpp, abi.cpp) with
  tests/sanitize/host_driver.cpp, which serves their HIP runtime calls from
  host memory and replaces each launch by a host loop that reaches exactly
  what the kernel reaches through the tile table -- an entry pointing
  outside a weight is a sanitizer report.
Leak checking is on: plans and their tables must be freed by
bfz_plan_destroy."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd_build, exe):
    b = subprocess.run(cmd_build, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out and "runtime error" not in out, out[-6000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _run(["gcc", "-std=gnu99", *SAN, "-ffp-contract=off", "-I" + os.path.join(ROOT, "oracle"),
                os.path.join(ROOT, "oracle", "oracle.c"),
                os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"], exe)
    assert "all checks passed" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_planner_and_abi_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "blockwise_fp8_zero_amd", "csrc")
    exe = str(tmp_path / "host_driver")
    out = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
                os.path.join(csrc, "plan.cpp"), os.path.join(csrc, "abi.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", exe], exe)
    assert "all checks passed" in out
