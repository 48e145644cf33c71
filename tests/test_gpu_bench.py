"""bench.py's output contract on the GPU: a short run on a small workload,
in a child process, prints one JSON line with every field the contract
names (metric, value, unit, n_gpus, steps, warmup, ms_per_step,
higher_is_better, scaling, vs_baseline, dtype, data, config.workload) and
the roofline, fold / unfold / transpose and parity objects, all sane."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_the_contract_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "moe_experts",
           "--steps", "3", "--warmup", "1", "--skip-configs"]
    print("[gpu-bench]", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=280)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    b = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert k in b, k
    assert b["n_gpus"] == 1 and b["steps"] == 3 and b["warmup"] == 1
    assert b["higher_is_better"] is True and b["scaling"] == "weak" and b["data"] == "synthetic"
    assert b["dtype"] == "f32" and b["unit"] == "elem/s"
    assert b["config"]["workload"].startswith("moe_experts")
    assert b["value"] > 0 and b["ms_per_step"] > 0
    # throughput and time agree: value counts the shard's elements per second
    assert abs(b["value"] * b["ms_per_step"] * 1e-3 - b["config"]["shard_elems"]) \
        < 1e-6 * b["config"]["shard_elems"]
    rf = b["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] < 1 and abs(rf["achieved"] / rf["peak"] - rf["frac"]) < 1e-9
    # the kernel cannot beat the whole step, nor HBM its peak
    assert b["step_kernel_ms"] <= b["ms_per_step"] * 1.001
    for k in ("pack", "unpack", "transpose_pow2"):
        assert 0 < b[k]["frac"] < 1 and b[k]["ms"] > 0, k
    par = b["parity"]
    assert par["headline"]["bit_exact"] and par["headline"]["code_mismatches"] == 0
    assert par["tiny"]["bit_exact"]
    dev = b["device"]
    assert dev["compute_units"] == 256 and "gfx950" in (dev["arch"] or ""), dev
    cb = b["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
