"""bench.py's contract checks that need no GPU (CPU only)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_timed_path_does_not_load_the_oracle():
    """Only the cpu_baseline leg may load the oracle: importing bench and the
    GPU workload driver it times must leave it unloaded."""
    code = ("import sys; import bench; import bench_workload; "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), "
            "sorted(m for m in sys.modules if 'oracle' in m)")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]


def test_traffic_is_reported_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    good = tmp_path / "step_kernel_good_traffic.md"
    stale = tmp_path / "step_kernel_stale_traffic.md"
    good.write_text(f"kernel_sha256: {bench.kernel_sha()}\ntraffic_bytes_per_call: 2.5e+10\n")
    stale.write_text("kernel_sha256: " + "0" * 64 + "\ntraffic_bytes_per_call: 2.5e+10\n")
    monkeypatch.setattr(bench, "traffic_file",
                        lambda kernel, workload: str(tmp_path / f"{kernel}_{workload}_traffic.md"))
    assert bench.measured_traffic("step_kernel", "good") == 2.5e10
    assert bench.measured_traffic("step_kernel", "stale") is None
    assert bench.measured_traffic("step_kernel", "missing") is None


def test_step_bytes_accounting():
    """The one-kernel step's algorithmic bytes: 30 B per element + 8 B per
    tile on full tiles (24 B of state, 4 B of gradient, the tile-major and the
    row-major code, scale_inv and the scale-grid cell); the fused route moves
    the unfold into a pass of its own, the unfused one the fold as well."""
    q, owned = 10, 9
    valid = 9 * 16384 - 100
    one, whole = bench.step_bytes(q, owned, valid, 9 * 128, "fused_unpack")
    assert one == whole == 24 * q * 16384 + 4 * valid + q * 16384 + 4 * q + valid + 4 * owned
    full, _ = bench.step_bytes(5, 5, 5 * 16384, 5 * 128, "fused_unpack")
    assert full == 30 * 5 * 16384 + 8 * 5
    step, whole = bench.step_bytes(q, owned, valid, 0, "fused")
    assert step == 24 * q * 16384 + 4 * valid + q * 16384 + 4 * q
    assert whole == step + owned * 16384 + valid + 8 * owned
    step, whole = bench.step_bytes(q, owned, valid, 0, "unfused")
    assert step == 29 * q * 16384 + 4 * q
    assert whole == step + owned * 16384 + valid + 8 * owned + 4 * valid + 4 * q * 16384


def test_kernel_hash_follows_code_not_comments(tmp_path, monkeypatch):
    """A comment or whitespace edit keeps the hash (the compiled kernels are
    the same); any change to the code changes it."""
    src = open(bench.KERNEL_SRC).read()
    base = bench.kernel_sha()
    variants = {"comment": src.replace("namespace bfz {", "namespace bfz {  // a note\n/* block\n note */", 1),
                "spaces": src.replace("\n", "\n   \n", 5),
                "code": src.replace("kStepLdsBytes = 96 * 1024", "kStepLdsBytes = 95 * 1024", 1)}
    assert variants["code"] != src
    got = {}
    for name, text in variants.items():
        f = tmp_path / f"{name}.hip"
        f.write_text(text)
        monkeypatch.setattr(bench, "KERNEL_SRC", str(f))
        got[name] = bench.kernel_sha()
    assert got["comment"] == base and got["spaces"] == base and got["code"] != base

