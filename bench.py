"""Benchmark of the block-wise FP8 ZeRO-1 shard step on one MI355X.

One step = the whole per-step path of one rank: fold its row-major FP32
grads into the tile layout, the AdamW + per-tile E4M3 requantization, and
the unfold of codes and scales into row-major FP8 weights plus the scale
grid.  --path picks how:
  fused_unpack (default): fold_adamw_fp8_step_unpack -- all of it in one
      kernel, writing the tile-major codes/scales (the all-gather payload)
      and the row-major FP8 weights/scale grids;
  fused_unpack_t: fold_adamw_fp8_step_unpack_t -- the same with power-of-two
      scales, also writing the transposed copy W^T and its group scales;
  fused:   fold_adamw_fp8_step, then unpack_fp8;
  unfused: pack_shard, adamw_fp8_step, unpack_fp8.
The split itself (the planner) runs once at set-up.
--layout picks how the FP32 state (master, m, v) sits in HBM:
  interleaved (default): one contiguous [master | m | v] block per tile
      and a 4 KiB gap (state_stride 50176), so each tile's updated state
      leaves as one write stream;
  separate: three tile-major arrays.

Default workload (the headline): the large shard -- 120 matrices of
4096x4096, 2.01B elements, D = 1, step t = 1000, 1% of the tiles all zero;
every output is written: the tile-major codes and scale_inv and the
row-major FP8 weights and scale grids.  Its inputs stay resident in HBM:
the timed steps continue at t = 1000, 1001, ... on the t = 1000 gradients
(never re-drawn inside the timed region).

Output: one JSON line.  value = shard elements per second of the whole
step (padded elements; on the headline workload every element is valid).
roofline = the step kernel's algorithmic HBM bytes per step (master, m, v
read and written: 24 B per element; the gradient read: 4 B per valid
element; the tile-major code: 1 B per element; scale_inv: 4 B per tile; the
row-major code: 1 B per valid element; the scale-grid cell: 4 B per owned
tile) over its mean time per step, measured with HIP events on the stream
the kernels run on.  A step is one launch per segment of at most 64
weights (two on the headline shard, same rate per tile), so bytes per step
over time per step equals bytes per launch over launch time; traffic =
the committed rocprofv3 FETCH_SIZE + WRITE_SIZE bytes per step of the same
kernel, while the kernel source still hashes as when they were taken.  After the timed region, outside it:
  configs: the other shard workloads (dense-LLM, MoE experts, ragged)
      through the same one-kernel step, each timed the same way;
  pack / unpack: pack_shard of the gradients and unpack_fp8 of the codes
      as passes of their own on the headline shard;
  transpose_pow2: the scaling-aware transpose on the headline shard;
  parity (oracle leg): sampled slots of the headline step and every slot
      of a tiny workload compared with the C oracle, counts reported;
  cpu_baseline (oracle leg): the C oracle on a bounded sample of the
      headline workload, on the host's cores.
"""
import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "AdamW+blockwise-FP8 requant elems/s and HBM GB/s (% of peak) on one MI355X"
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published peak
KERNEL_OF_PATH = {"fused_unpack": "fold_step_unfold_kernel",
                  "fused_unpack_t": "fold_step_unfold_t_kernel", "fused": "fold_step_kernel",
                  "unfused": "step_kernel"}
KERNEL_SRC = os.path.join(ROOT, "blockwise_fp8_zero_amd", "csrc", "kernels.hip")
OTHER_CONFIGS = ("dense_llm", "moe_experts", "ragged")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def traffic_file(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")


def kernel_sha():
    """sha256 of kernels.hip's code: comments removed and whitespace runs
    collapsed, so that a comment edit does not orphan the committed counter
    summaries while any change to the code does."""
    with open(KERNEL_SRC) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes of `kernel` per call of its entry point (all launch segments
    of one step or pass) on `workload`, from its committed rocprofv3 PMC
    summary, if that was taken on the current kernel source; else None."""
    path = traffic_file(kernel, workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_sha256:\s*([0-9a-f]{64})", text)
    tb = re.search(r"traffic_bytes_per_call:\s*([0-9.eE+]+)", text)
    if not sha or not tb or sha.group(1) != kernel_sha():
        return None
    return float(tb.group(1))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def step_bytes(q, owned, valid, valid_cols, path, tile_codes=True):
    """Algorithmic HBM bytes of one step of `path` over a shard of q slots
    (owned tiles, valid elements, and valid_cols = the W^T rows of the owned
    tiles), as (step kernel bytes, whole-step bytes incl. separate passes)."""
    elems = q * 16384
    grad = 4 * (elems if path == "unfused" else valid)
    b = 24 * elems + grad
    if tile_codes:
        b += elems + 4 * q
    if path in ("fused_unpack", "fused_unpack_t"):
        b += valid + 4 * owned
    if path == "fused_unpack_t":
        b += valid + 4 * valid_cols
    whole = b
    if path in ("fused", "unfused"):
        whole += owned * 16384 + valid + 8 * owned   # unpack_fp8
    if path == "unfused":
        whole += 4 * valid + 4 * elems                # pack_shard of the gradients
    return b, whole


def shard_counts(g):
    owned = g.table[:g.owned]
    return g.q, g.owned, int((owned[:, 4] * owned[:, 5]).sum()), int(owned[:, 5].sum())


class no_gc:
    """Python's garbage collector held off from before the warm-up until the
    timed loop is done: a collection pause on the host while the device
    queue runs dry would be timed as device time, and one between warm-up
    and timing would let the device idle (and its clocks drop) before the
    first timed step.  The collection runs first, before any warm-up."""

    def __enter__(self):
        gc.collect()
        gc.disable()

    def __exit__(self, *exc):
        gc.enable()


def timed(stream, fn, n):
    """Mean ms of fn() over n calls, HIP events on `stream` around the run,
    after one untimed call."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with no_gc():
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def setup(w, path="fused_unpack", pow2=False, layout="interleaved"):
    """Device state of workload w, its prior steps taken, gradients of the
    measured step drawn: ready for the timed steps."""
    from bench_workload import GpuWorkload
    transposed = path == "fused_unpack_t"
    one_kernel = path in ("fused_unpack", "fused_unpack_t")
    g = GpuWorkload(w, mode="fused_unpack" if one_kernel else path, pow2=pow2 or transposed,
                    transposed=transposed, layout=layout)
    g.tile_codes = True
    g.load_state()
    if w.steps[:-1]:
        g.run_steps(w.steps[:-1])
    g.draw_grads(w.measured_step)
    return g


def run_steps(g, path, steps, warmup, t_first, stream, fp8=None, sc=None):
    """W untimed steps, then K timed ones; HIP events around the step
    kernel, the fold and the unfold of every timed step."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    t = t_first

    def one(t, e=None):
        if path == "unfused":
            e and e[2].record(stream)
            g.pack_grads()
            e and e[3].record(stream)
        e and e[0].record(stream)
        if path == "unfused":
            g.step(t)
        elif path == "fused":
            g.fold_step(t)
        else:
            g.fold_step_unpack(t)
        e and e[1].record(stream)
        if path in ("fused", "unfused"):
            e and e[4].record(stream)
            g.unpack(fp8, sc)
            e and e[5].record(stream)

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with no_gc():
        for _ in range(warmup):
            one(t)
            t += 1
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(steps):
            one(t, ev[k])
            t += 1
        end.record(stream)
        torch.cuda.synchronize()
    kms = [e[0].elapsed_time(e[1]) for e in ev]
    res = {"ms_per_step": start.elapsed_time(end) / steps,
           "kernel_ms": sum(kms) / steps,
           "kernel_ms_min": min(kms) if kms else None,
           "kernel_ms_max": max(kms) if kms else None,
           "pack_ms": (sum(e[2].elapsed_time(e[3]) for e in ev) / steps
                       if path == "unfused" else None),
           "unpack_ms": (sum(e[4].elapsed_time(e[5]) for e in ev) / steps
                         if path in ("fused", "unfused") else None),
           "t_next": t}
    return res


def pass_stats(ms, algo, traffic=None):
    gbps = algo / (ms * 1e-3) / 1e9
    return {"ms": ms, "algorithmic_bytes": algo, "GBps": gbps, "frac": gbps / HBM_PEAK_GBPS,
            "traffic": traffic}


def time_pack_unpack(g, steps, stream):
    """pack_shard of the row-major gradients into a tile-major buffer, and
    unpack_fp8 of the step's codes and scales, each timed over `steps`
    launches on the headline shard."""
    import torch

    import blockwise_fp8_zero_amd as bfz
    q, owned, valid, _ = shard_counts(g)
    g.grad = torch.empty(q * bfz.TILE_ELEMS, dtype=torch.float32, device=g.device)
    g.pack_grads()
    fp8, sc = (g.out_fp8, g.out_scale) if g.out_fp8 is not None else g.alloc_rowmajor_out()
    g.unpack(fp8, sc)
    torch.cuda.synchronize()
    pack_ms = timed(stream, g.pack_grads, steps)
    unpack_ms = timed(stream, lambda: g.unpack(fp8, sc), steps)
    g.grad = None
    torch.cuda.empty_cache()
    return (pass_stats(pack_ms, 4 * valid + 4 * q * 16384, measured_traffic("pack_kernel", g.w.name)),
            pass_stats(unpack_ms, owned * 16384 + valid + 8 * owned,
                       measured_traffic("unpack_kernel", g.w.name)))


def time_transpose(g, t, steps, stream):
    """One power-of-two step (so every tile scale is a power of two), then
    bfz_transpose_pow2 of the shard timed over `steps` launches: W^T codes
    and per-group power-of-two scales by exponent edits."""
    import torch

    import blockwise_fp8_zero_amd as bfz
    pow2_was = g.pow2
    g.pow2 = True
    g.apply(t)
    g.pow2 = pow2_was
    dims = g.w.dims
    dt = [None] * len(dims)
    ds = [None] * len(dims)
    for p in g.touched:
        E, H, W = dims[p]
        dt[p] = torch.empty(E * W * H, dtype=torch.uint8, device="cuda")
        ds[p] = torch.empty(E * W * (-(-H // 128)), dtype=torch.float32, device="cuda")
    bfz.transpose_pow2(g.plan, g.codes, g.scale_inv, dt, ds)
    torch.cuda.synchronize()
    ms = timed(stream, lambda: bfz.transpose_pow2(g.plan, g.codes, g.scale_inv, dt, ds), steps)
    q, owned, valid, valid_cols = shard_counts(g)
    # read: tile codes + scale; write: W^T codes of the valid elements + one
    # scale per valid column of every owned tile
    algo = q * bfz.TILE_ELEMS + 4 * q + valid + 4 * valid_cols
    del dt, ds
    torch.cuda.empty_cache()
    out = pass_stats(ms, algo, measured_traffic("transpose_pow2_kernel", g.w.name))
    out["kernel"] = "transpose_pow2_kernel"
    return out


def counter_reference_copy():
    """A plain 1 GiB device copy (the runtime's copy kernel), once, outside
    the timed region: the kernel of known size that rocprofv3's HBM byte
    counters are scaled by."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def sampled_gpu_slots(g, n_random=24):
    """The GPU's state, codes and scales of a sample of slots after the
    measured step (first, last, weight boundaries, edges, zero tiles and a
    seeded random draw), read back to the host for the oracle leg."""
    from bench_workload import sample_slots
    slots = sample_slots(g.w, g.table, g.q, g.owned, n_random=n_random)
    return slots, g.tiles(slots)


def oracle_leg(w, gpu_sample, tiny_gpu):
    """Parity counts of the sampled headline slots and of the tiny workload
    against the oracle.  With cpu_baseline below, this is the CPU-baseline
    leg of the run, the only part of bench.py that loads the oracle (both
    are skipped by --skip-cpu-baseline)."""
    import numpy as np

    import oracle
    from tests.compare import compare
    from tests.oracle_run import oracle_slots

    out = {}
    slots, gpu = gpu_sample
    ora = oracle_slots(w, slots)
    rep = compare(gpu, ora)
    out["headline"] = {"workload": w.name, "slots_compared": len(slots),
                       "elements": len(slots) * oracle.TILE_ELEMS, "ok": rep["ok"],
                       "bit_exact": rep["exact"], "code_mismatches": rep["codes_mismatch"],
                       "midpoint_exceptions": rep["codes_mismatch_near_midpoint"],
                       "near_midpoint_elems": rep["near_midpoint_elems"],
                       "fp32_out_of_tolerance": rep["master_bad"] + rep["m_bad"] + rep["v_bad"],
                       "scale_out_of_tolerance": rep["scale_bad"]}
    tw, tg, tfp8 = tiny_gpu
    tslots = list(range(len(tg["scale_inv"])))
    tora = oracle_slots(tw, tslots)
    trep = compare(tg, tora)
    q, owned, table = oracle.plan(tw.dims, tw.D, tw.rank)
    E, H, W = tw.dims[0]
    o8 = np.zeros((E, H, W), dtype=np.uint8)
    osc = np.zeros((E, -(-H // 128), -(-W // 128)), dtype=np.float32)
    oracle.unpack(tw.dims, tora["codes"].reshape(-1), tora["scale_inv"], table, [o8], [osc])
    unpack_exact = bool(np.array_equal(tfp8[0].reshape(-1), o8.reshape(-1))
                        and np.array_equal(tfp8[1].reshape(-1), osc.reshape(-1)))
    out["tiny"] = {"workload": tw.name, "slots_compared": len(tslots), "steps": len(tw.steps),
                   "ok": trep["ok"], "bit_exact": trep["exact"],
                   "code_mismatches": trep["codes_mismatch"],
                   "midpoint_exceptions": trep["codes_mismatch_near_midpoint"],
                   "row_major_unpack_exact": unpack_exact}
    return out


def cpu_baseline(w, target_s=10.0):
    """The C oracle (fold of the grads, AdamW + requant, unfold) on a slab of
    the workload's first weight, 1024 rows of it (8 tile rows), stepped
    repeatedly by every host thread for about target_s seconds."""
    import ctypes as C
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth
    from synth import workloads as WL

    threads = min(16, os.cpu_count() or 1)
    E, H, W = 1, 1024, w.dims[0][2]
    dims = np.array([[E, H, W]], dtype=np.int64)
    q, owned, table = oracle.plan(dims, 1, 0)
    n = q * oracle.TILE_ELEMS
    # the slab's own inputs: the workload's recipes for its first weight
    rect = {k: synth.fill_rect_host(w.recipe(k, 0, w.measured_step), 0, 0, H, 0, W)
            for k in (WL.MASTER, WL.GRAD, WL.MOM1, WL.MOM2)}
    grad_rm = rect[WL.GRAD]
    L = oracle.lib()
    hp = oracle.hparams(step=w.measured_step, **WL.HP)
    P = C.c_void_p

    def ptr(a):
        return a.ctypes.data_as(P)

    def one_pass(state):
        g_tiles, p, m, v, codes, sc, out8, outsc = state
        srcs = (P * 1)(grad_rm.ctypes.data)
        L.ora_pack(ptr(dims), 1, C.cast(srcs, P), ptr(table), q, ptr(g_tiles))
        L.ora_step(ptr(p), ptr(g_tiles), ptr(m), ptr(v), q, C.byref(hp), ptr(codes), ptr(sc),
                   None, 1e-6)
        d8 = (P * 1)(out8.ctypes.data)
        ds = (P * 1)(outsc.ctypes.data)
        L.ora_unpack(ptr(dims), 1, ptr(codes), ptr(sc), ptr(table), q, C.cast(d8, P), C.cast(ds, P))

    def new_state():
        fold = [oracle.pack(dims, [np.ascontiguousarray(rect[k].reshape(E, H, W))], table)
                for k in (WL.MASTER, WL.MOM1, WL.MOM2)]
        return [np.empty(n, np.float32), fold[0], fold[1], fold[2], np.empty(n, np.uint8),
                np.empty(q, np.float32), np.empty(E * H * W, np.uint8), np.empty(q, np.float32)]

    # calibrate the number of passes on one thread (the second pass: the
    # first one takes the page faults of the fresh buffers)
    st = new_state()
    one_pass(st)
    t0 = time.perf_counter()
    one_pass(st)
    per_pass = time.perf_counter() - t0
    passes = max(1, int(round(target_s / per_pass)))
    # a one-thread figure over a 1 GiB tile subset (16384 tiles of master,
    # the slab's state in separate copies, so the data lives in DRAM, not in
    # the caches), one pass over each copy
    copies = [new_state() for _ in range(max(1, 16384 // q))]
    for c in copies:  # take the page faults of the fresh buffers now
        for k in (0, 4, 5, 6, 7):
            c[k].fill(0)
    t0 = time.perf_counter()
    for c in copies:
        one_pass(c)
    one_thread = len(copies) * n / (time.perf_counter() - t0)
    one_thread_gib = len(copies) * n * 4 / 2 ** 30
    del copies
    states = [new_state() for _ in range(threads)]

    def work(k, count):
        for _ in range(count):
            one_pass(states[k])

    with ThreadPoolExecutor(max_workers=threads) as ex:
        # one untimed pass per thread first: it takes the page faults of the
        # freshly allocated buffers, which serialize across threads
        list(ex.map(lambda k: work(k, 1), range(threads)))
        t0 = time.perf_counter()
        list(ex.map(lambda k: work(k, passes), range(threads)))
        dt = time.perf_counter() - t0
    elems = threads * passes * n
    return {"value": elems / dt, "unit": "elem/s", "cores": threads, "kind": "oracle",
            "one_thread_value": one_thread,
            "one_thread_sample": f"one thread, one pass over {one_thread_gib:.2f} GiB of master "
                                 f"(the slab's state in {16384 // q} copies)",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"fold + AdamW/E4M3 step + unfold of a {H}x{W} slab ({q} tiles, "
                      f"{n / 1e6:.1f}M elements) of the first weight of the {w.name} workload, "
                      f"its own master/m/v/grad draws, at t={w.measured_step}; {passes} passes "
                      f"on each of {threads} threads, {dt:.1f} s wall",
            "seconds": round(dt, 2)}


def tiny_gpu_run():
    """The tiny workload (one 256x384 weight, 3 steps) through the same
    one-kernel step and interleaved layout; results read back for the
    oracle leg's parity counts."""
    from bench_workload import GpuWorkload
    from synth import workloads as WL
    w = WL.tiny()
    g = GpuWorkload(w, mode="fused_unpack", layout="interleaved")
    g.load_state()
    g.run_steps()
    tiles = g.tiles(list(range(g.q)))
    fp8, sc = g.rowmajor()
    return w, tiles, (fp8[0].cpu().numpy(), sc[0].cpu().numpy())


def config_line(w, args, stream):
    """One of the other shard workloads through the default one-kernel step,
    timed like the headline (its own set-up, warm-up and timed steps); a
    short shard takes more steps than K, enough for about 50 ms of timed
    work at the headline's rate, so one host or device hiccup weighs less."""
    import torch
    t0 = time.perf_counter()
    g = setup(w)
    q, owned, valid, valid_cols = shard_counts(g)
    algo, _ = step_bytes(q, owned, valid, valid_cols, "fused_unpack")
    est_ms = algo / 6.3e12 * 1e3
    steps = max(args.steps, int(50.0 / est_ms))
    warmup = max(args.warmup, steps // 4)
    r = run_steps(g, "fused_unpack", steps, warmup, w.measured_step, stream)
    elems = q * 16384
    out = {"workload": f"{w.name}: {w.description}", "shard_tiles": q, "shard_elems": elems,
           "valid_elems": valid, "D": w.D, "rank": w.rank, "steps": steps, "warmup": warmup,
           "ms_per_step": r["ms_per_step"],
           "value": elems / (r["ms_per_step"] * 1e-3),
           "valid_elems_per_s": valid / (r["ms_per_step"] * 1e-3),
           "step_kernel_ms": r["kernel_ms"],
           "step_kernel_ms_min_max": [r["kernel_ms_min"], r["kernel_ms_max"]],
           "algorithmic_bytes_per_step": algo,
           "roofline_frac": algo / (r["kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "traffic": measured_traffic("fold_step_unfold_kernel", w.name)}
    del g
    torch.cuda.empty_cache()
    log(f"config {w.name}: {r['ms_per_step']:.4f} ms/step, frac {out['roofline_frac']:.4f} "
        f"({time.perf_counter() - t0:.1f} s)")
    return out


def device_info():
    """The GPU the line was measured on (boxes of one model differ by a few
    percent in these numbers): name, architecture, CUs, memory, and the
    device's PCI bus id so that runs on one board can be told apart."""
    import torch
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "memory_GiB": round(p.total_memory / 2 ** 30, 1)}
    for key in ("pci_bus_id", "pci_device_id", "pci_domain_id"):
        if hasattr(p, key):
            info[key] = getattr(p, key)
    return info


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large",
                    choices=["large", "dense_llm", "ragged", "moe_experts", "tiny"])
    ap.add_argument("--skip-cpu-baseline", action="store_true",
                    help="skip the oracle leg (CPU baseline and parity counts)")
    ap.add_argument("--skip-configs", action="store_true",
                    help="do not time the other shard workloads after the headline")
    ap.add_argument("--skip-passes", action="store_true",
                    help="do not time pack / unpack / transpose / copy after the steps")
    ap.add_argument("--path", default="fused_unpack", choices=list(KERNEL_OF_PATH),
                    help="which entry points make up a step (see the module docstring)")
    ap.add_argument("--pow2", action="store_true",
                    help="power-of-two tile scales in the timed steps")
    ap.add_argument("--layout", default="interleaved", choices=["interleaved", "separate"],
                    help="FP32 state layout (see the module docstring)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import blockwise_fp8_zero_amd as bfz
    from bench_workload import launch_segments
    from synth import workloads as WL

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    w = WL.BY_NAME[args.workload]()
    log(f"workload {w.name}: {w.description}")
    t0 = time.perf_counter()
    g = setup(w, args.path, args.pow2, args.layout)
    one_kernel = args.path in ("fused_unpack", "fused_unpack_t")
    fp8, sc = g.alloc_rowmajor_out() if not one_kernel else (None, None)
    # the measured step itself, once, from the seeded state: a sample of its
    # slots goes to the oracle leg for the parity counts
    first = run_steps(g, args.path, 1, 0, w.measured_step, stream, fp8, sc)
    gpu_sample = None if args.skip_cpu_baseline else sampled_gpu_slots(g)
    counter_reference_copy()
    log(f"set-up {time.perf_counter() - t0:.1f} s; q={g.q} tiles, owned={g.owned}")

    r = run_steps(g, args.path, args.steps, args.warmup, first["t_next"], stream, fp8, sc)
    q, owned, valid, valid_cols = shard_counts(g)
    kernel = KERNEL_OF_PATH[args.path]
    algo, whole = step_bytes(q, owned, valid, valid_cols, args.path)
    elems = q * bfz.TILE_ELEMS
    achieved = algo / (r["kernel_ms"] * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": elems / (r["ms_per_step"] * 1e-3),
        "unit": "elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "shard_tiles": q,
            "shard_elems": elems,
            "valid_elems": valid,
            "value_counts": "shard elements incl. padding slots and edge padding "
                            "(valid_elems_per_s counts the weights' own elements)",
            "D": w.D,
            "rank": w.rank,
            "first_timed_step_t": first["t_next"] + args.warmup,
            "state_layout": {"interleaved": "one [master | m | v] block per tile "
                                            "and a 4 KiB gap (state_stride 50176)",
                             "separate": "three tile-major arrays"}[args.layout],
            "step_path": {"unfused": "pack_shard(grad) + adamw_fp8_step + unpack_fp8",
                          "fused": "fold_adamw_fp8_step + unpack_fp8",
                          "fused_unpack": "fold_adamw_fp8_step_unpack",
                          "fused_unpack_t": "fold_adamw_fp8_step_unpack_t (power-of-two scales, "
                                            "plus the transposed copy W^T)"}[args.path],
            "outputs": "tile-major codes + scale_inv (the all-gather payload) and row-major "
                       "FP8 weights + scale grids",
        },
        "valid_elems_per_s": valid / (r["ms_per_step"] * 1e-3),
        "step_hbm_GBps": whole / (r["ms_per_step"] * 1e-3) / 1e9,
        "step_hbm_frac": whole / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "step_kernel_ms": r["kernel_ms"],
        "step_kernel_ms_min_max": [r["kernel_ms_min"], r["kernel_ms_max"]],
        "step_kernel_elems_per_s": elems / (r["kernel_ms"] * 1e-3),
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic(kernel, w.name),
            "algorithmic_bytes_per_step": algo,
            "launches_per_step": launch_segments(g.table, owned, q),
        },
        "cpu_baseline": None,
        "parity": None,
        "pack": None,
        "unpack": None,
        "transpose_pow2": None,
        "configs": None,
        "device": device_info(),
    }
    if r["pack_ms"] is not None:
        out["pack"] = pass_stats(r["pack_ms"], 4 * valid + 4 * elems)
    if r["unpack_ms"] is not None:
        out["unpack"] = pass_stats(r["unpack_ms"], owned * 16384 + valid + 8 * owned)
    if not args.skip_passes:
        if out["pack"] is None or out["unpack"] is None:
            p_, u_ = time_pack_unpack(g, args.steps, stream)
            out["pack"] = out["pack"] or p_
            out["unpack"] = out["unpack"] or u_
        out["transpose_pow2"] = time_transpose(g, r["t_next"], args.steps, stream)
    # memory returned to the HIP runtime: each config below gets fresh allocations (tensors
    # carved out of the headline's cached blocks measured up to 10% slower)
    del g
    torch.cuda.empty_cache()
    if not args.skip_configs:
        out["configs"] = {n: config_line(WL.BY_NAME[n](), args, stream)
                          for n in OTHER_CONFIGS if n != w.name}
    if not args.skip_cpu_baseline:
        tiny = tiny_gpu_run()
        log("oracle leg: parity counts and cpu baseline ...")
        out["parity"] = oracle_leg(w, gpu_sample, tiny)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
