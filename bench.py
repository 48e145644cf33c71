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
      (state_stride 49152), so each tile's updated state leaves as one
      write stream;
  separate: three tile-major arrays.

Default workload: the dense-LLM rank shard -- 32 layers x {4 of 4096x4096,
2 of 4096x11008, 1 of 11008x4096}, D = 8, rank 0: 49408 tiles, 809.5M
elements.  Its moments are warm from 10 prior steps (t = 1..10, fresh
N(0, 1e-3) grads each); the timed steps continue at t = 11, 12, ... on the
t = 11 gradients, which stay resident in HBM (inputs are never re-drawn
inside the timed region).

Output: one JSON line.  value = shard elements per second of the whole
step.  roofline = the step kernel's algorithmic HBM bytes per launch
(29 B per element + 4 B per tile, plus 1 B per element + 4 B per tile for
the row-major codes and scales in the one-kernel path; gradient reads and
row-major writes count valid elements) over its mean launch time, measured
with HIP events on the stream the kernels run on.  pack / unpack = the fold
and the unfold timed the same way where they run as passes of their own
(unfused / fused routes).  cpu_baseline = the C oracle on a bounded sample
of the same workload, on the host's cores.
"""
import argparse
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
STEP_BYTES_PER_ELEM = 29          # read p, g, m, v (16) + write p, m, v (12) + code (1)
STEP_BYTES_PER_TILE = 4           # scale_inv
PACK_BYTES_PER_ELEM = 8           # read grad + write tile
UNPACK_BYTES_PER_ELEM = 2         # read code + write code
UNPACK_BYTES_PER_TILE = 8         # read + write scale
TRAFFIC_FILES = {k: os.path.join(ROOT, "profiles", f"{k}_dense_llm_traffic.md")
                 for k in ("fold_step_unfold_kernel", "fold_step_kernel", "step_kernel",
                           "transpose_pow2_kernel", "fold_step_unfold_t_kernel")}
KERNEL_OF_PATH = {"fused_unpack": "fold_step_unfold_kernel",
                  "fused_unpack_t": "fold_step_unfold_t_kernel", "fused": "fold_step_kernel",
                  "unfused": "step_kernel"}
KERNEL_SRC = os.path.join(ROOT, "blockwise_fp8_zero_amd", "csrc", "kernels.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


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


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from its committed rocprofv3 PMC
    summary, if that was taken on the current kernel source; else None."""
    path = TRAFFIC_FILES[kernel]
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_sha256:\s*([0-9a-f]{64})", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
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


def cpu_baseline(w, target_s=10.0):
    """The C oracle (fold of the grads, AdamW + requant, unfold) on a slab of
    the workload's first weight, 1024 x 4096 (256 tiles), stepped repeatedly
    by every host thread for about target_s seconds."""
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
    master_rm = synth.fill_rect_host(w.recipe(WL.MASTER, 0), 0, 0, H, 0, W)
    grad_rm = synth.fill_rect_host(w.recipe(WL.GRAD, 0, w.measured_step), 0, 0, H, 0, W)
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
        srcs = [np.ascontiguousarray(master_rm.reshape(E, H, W))]
        p = oracle.pack(dims, srcs, table)
        return [np.empty(n, np.float32), p, np.zeros(n, np.float32), np.zeros(n, np.float32),
                np.empty(n, np.uint8), np.empty(q, np.float32), np.empty(E * H * W, np.uint8),
                np.empty(q, np.float32)]

    # calibrate the number of passes on one thread (the second pass: the
    # first one takes the page faults of the fresh buffers)
    st = new_state()
    one_pass(st)
    t0 = time.perf_counter()
    one_pass(st)
    per_pass = time.perf_counter() - t0
    passes = max(1, int(round(target_s / per_pass)))
    # a one-thread figure over a 1 GiB tile subset (16384 tiles of master,
    # the slab's state in 64 separate copies, so the data lives in DRAM, not
    # in the caches), one pass over each copy
    copies = [new_state() for _ in range(max(1, 16384 // q))]
    for c in copies:  # take the page faults of the fresh buffers now
        for k, a in enumerate(c):
            if k != 1:  # c[1] holds the folded master
                a.fill(0)
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
            "sample": f"fold + AdamW/E4M3 step + unfold of a {H}x{W} slab (256 tiles, "
                      f"{n / 1e6:.1f}M elements) of the first dense-LLM weight at t="
                      f"{w.measured_step}, {passes} passes on each of {threads} threads, "
                      f"{dt:.1f} s wall",
            "seconds": round(dt, 2)}


def time_transpose(g, t, steps, stream):
    """One power-of-two step (so every tile scale is a power of two), then
    bfz_transpose_pow2 of the shard timed over `steps` launches: W^T codes
    and per-group power-of-two scales by exponent edits."""
    import torch

    import blockwise_fp8_zero_amd as bfz
    pow2_was, tile_codes_was = g.pow2, g.tile_codes
    g.pow2, g.tile_codes = True, True  # the transpose reads the tile-major codes
    g.apply(t)
    g.pow2, g.tile_codes = pow2_was, tile_codes_was
    dims = g.w.dims
    dt = [None] * len(dims)
    ds = [None] * len(dims)
    for p in g.touched:
        E, H, W = dims[p]
        dt[p] = torch.empty(E * W * H, dtype=torch.uint8, device="cuda")
        ds[p] = torch.empty(E * W * (-(-H // 128)), dtype=torch.float32, device="cuda")
    bfz.transpose_pow2(g.plan, g.codes, g.scale_inv, dt, ds)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        bfz.transpose_pow2(g.plan, g.codes, g.scale_inv, dt, ds)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    owned = g.table[:g.owned]
    valid = int((owned[:, 4] * owned[:, 5]).sum())
    # read: tile codes + scale; write: W^T codes of the valid elements + one
    # scale per valid column of every owned tile
    algo = g.q * bfz.TILE_ELEMS + 4 * g.q + valid + 4 * int(owned[:, 5].sum())
    del dt, ds
    traffic = measured_traffic("transpose_pow2_kernel") if g.w.name == "dense_llm" else None
    return {"kernel": "transpose_pow2_kernel", "ms": ms, "algorithmic_bytes": algo,
            "GBps": algo / (ms * 1e-3) / 1e9, "frac": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "traffic": traffic}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_llm",
                    choices=["dense_llm", "ragged", "moe_experts", "large", "tiny"])
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--path", default="fused_unpack", choices=list(KERNEL_OF_PATH),
                    help="which entry points make up a step (see the module docstring)")
    ap.add_argument("--pow2", action="store_true",
                    help="power-of-two tile scales in the timed steps (bfz_adamw.scale_pow2)")
    ap.add_argument("--skip-transpose", action="store_true",
                    help="do not time bfz_transpose_pow2 after the steps")
    ap.add_argument("--layout", default="interleaved", choices=["interleaved", "separate"],
                    help="FP32 state layout (see the module docstring)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import blockwise_fp8_zero_amd as bfz
    from synth import workloads as WL
    from bench_workload import GpuWorkload

    torch.cuda.set_device(0)
    w = WL.BY_NAME[args.workload]()
    log(f"workload {w.name}: {w.description}")
    t0 = time.perf_counter()
    # fused_unpack_t: the one-kernel step with power-of-two scales that also
    # writes the transposed copy W^T
    transposed = args.path == "fused_unpack_t"
    one_kernel = args.path in ("fused_unpack", "fused_unpack_t")
    g = GpuWorkload(w, mode="fused_unpack" if one_kernel else args.path,
                    pow2=args.pow2 or transposed, transposed=transposed, layout=args.layout)
    # a lone rank (D = 1) gathers nothing: its one-kernel step writes only
    # the row-major FP8 weights and scale grids, not the tile-major copy
    lone = one_kernel and w.D == 1
    g.load_state()
    prior = w.steps[:-1]
    if prior:
        g.run_steps(prior)
    g.draw_grads(w.measured_step)
    fp8, sc = g.alloc_rowmajor_out() if not one_kernel else (None, None)
    # a plain 1 GiB device copy, outside the timed region: the reference
    # kernel of known size for scaling the HBM byte counters
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    del a, b
    torch.cuda.synchronize()
    log(f"set-up {time.perf_counter() - t0:.1f} s; q={g.q} tiles, owned={g.owned}")

    stream = torch.cuda.current_stream()
    t_next = w.measured_step

    def one_step(t, ev=None):
        # ev: HIP events around the step kernel (0, 1), the fold (2, 3) and
        # the unfold (4, 5), recorded on the stream the kernels run on
        if args.path == "unfused":
            if ev is not None:
                ev[2].record(stream)
            g.pack_grads()
            if ev is not None:
                ev[3].record(stream)
        if ev is not None:
            ev[0].record(stream)
        if args.path == "unfused":
            g.step(t)
        elif args.path == "fused":
            g.fold_step(t)
        else:
            g.fold_step_unpack(t)
        if ev is not None:
            ev[1].record(stream)
        if not one_kernel:
            if ev is not None:
                ev[4].record(stream)
            g.unpack(fp8, sc)
            if ev is not None:
                ev[5].record(stream)

    g.tile_codes = not lone
    for _ in range(args.warmup):
        one_step(t_next)
        t_next += 1
    torch.cuda.synchronize()

    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(6)) for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        one_step(t_next, evs[k])
        t_next += 1
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    step_kernel_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    pack_ms = (sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
               if args.path == "unfused" else None)
    unpack_ms = (sum(e[4].elapsed_time(e[5]) for e in evs) / args.steps
                 if not one_kernel else None)
    ms_per_step = total_ms / args.steps

    elems = g.q * bfz.TILE_ELEMS
    valid = int((g.table[:g.owned, 4] * g.table[:g.owned, 5]).sum())
    kernel = KERNEL_OF_PATH[args.path]
    # fused kernels read the gradient of valid elements only
    grad_elems = elems if args.path == "unfused" else valid
    # master, m, v read and written (24 B), the gradient read (4 B, valid
    # elements only when read row-major), the tile-major code and scale
    algo_bytes = (STEP_BYTES_PER_ELEM - 5) * elems + 4 * grad_elems
    if not lone:
        algo_bytes += elems + STEP_BYTES_PER_TILE * g.q
    if one_kernel:
        # row-major codes of the valid elements and the scale-grid cells
        algo_bytes += valid + 4 * g.owned
    if transposed:
        # W^T codes of the valid elements, one scale per W^T row group
        algo_bytes += valid + 4 * int(g.table[:g.owned, 5].sum())
    achieved = algo_bytes / (step_kernel_ms * 1e-3) / 1e9
    whole_bytes = algo_bytes
    if not one_kernel:
        whole_bytes += UNPACK_BYTES_PER_ELEM * elems + UNPACK_BYTES_PER_TILE * g.q
    if args.path == "unfused":
        whole_bytes += PACK_BYTES_PER_ELEM * elems
    traffic = measured_traffic(kernel) if w.name == "dense_llm" and kernel in TRAFFIC_FILES else None
    transpose = None
    if not args.skip_transpose:
        transpose = time_transpose(g, t_next, args.steps, stream)

    def pass_stats(ms, algo):
        if ms is None:
            return None
        gbps = algo / (ms * 1e-3) / 1e9
        return {"ms": ms, "algorithmic_bytes": algo, "GBps": gbps, "frac": gbps / HBM_PEAK_GBPS}

    out = {
        "metric": METRIC,
        "value": elems / (ms_per_step * 1e-3),
        "unit": "elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "shard_tiles": g.q,
            "shard_elems": elems,
            "valid_elems": valid,
            "D": w.D,
            "rank": w.rank,
            "first_timed_step_t": w.measured_step + args.warmup,
            "state_layout": {"interleaved": "one [master | m | v] block per tile "
                                            "(state_stride 49152)",
                             "separate": "three tile-major arrays"}[args.layout],
            "step_path": {"unfused": "pack_shard(grad) + adamw_fp8_step + unpack_fp8",
                          "fused": "fold_adamw_fp8_step + unpack_fp8",
                          "fused_unpack": "fold_adamw_fp8_step_unpack",
                          "fused_unpack_t": "fold_adamw_fp8_step_unpack_t (power-of-two scales, "
                                            "plus the transposed copy W^T)"}[args.path]
                         + (" (row-major output only: D = 1)" if lone else ""),
        },
        "valid_elems_per_s": valid / (ms_per_step * 1e-3),
        "step_hbm_GBps": whole_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_hbm_frac": whole_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "step_kernel_ms": step_kernel_ms,
        "step_kernel_elems_per_s": elems / (step_kernel_ms * 1e-3),
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": algo_bytes,
        },
        "cpu_baseline": None,
        "transpose_pow2": transpose,
        # the fold and the unfold as passes of their own (unfused / fused
        # routes): fold reads the valid gradient elements and writes whole
        # tiles; unfold reads the owned tiles' codes and scales and writes
        # the valid codes and the scale-grid cells
        "pack": pass_stats(pack_ms, 4 * valid + 4 * elems),
        "unpack": pass_stats(unpack_ms, g.owned * bfz.TILE_ELEMS + valid + 8 * g.owned),
    }
    if not args.skip_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
