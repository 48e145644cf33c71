"""GPU parity of the HIP path against the oracle (needs an MI355X).

Every case prints its name, workload and seed before touching the GPU.
Sizes: the tiny and ragged workloads are compared element by element on
every slot; the dense-LLM, MoE and large workloads run at full size in
the launch configuration the benchmark times, and a sample of slots
(first, last, padding, ragged edges, weight boundaries, zero tiles and a
seeded random set) is recomputed by the oracle from regenerated inputs.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import blockwise_fp8_zero_amd as bfz
import oracle
from synth import workloads as WL
from tests.compare import compare
from bench_workload import GpuWorkload
from tests.oracle_run import oracle_slots, sample_slots

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _check(gpu, ora, what):
    rep = compare(gpu, ora)
    _say(what, {k: v for k, v in rep.items() if k != "fail"})
    assert rep["ok"], (what, rep["fail"])
    return rep


MODES = list(GpuWorkload.MODES)


LAYOUTS = list(GpuWorkload.LAYOUTS)
# the state layout bench.py times (one [master | m | v] block per tile)
BENCH_LAYOUT = "interleaved"


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("mode", MODES)
def test_tiny_every_step_every_slot(mode, layout):
    w = WL.tiny()
    _say("tiny: 256x384, 3 steps, seed", w.seed, "mode", mode, "layout", layout)
    g = GpuWorkload(w, mode=mode, layout=layout)
    g.load_state()
    slots = list(range(g.q))
    for k, t in enumerate(w.steps):
        g.run_steps([t])
        ora = oracle_slots(w, slots, steps=w.steps[:k + 1])
        rep = _check(g.tiles(slots), ora, f"tiny after t={t}")
        assert rep["exact"], "the step is expected to be bit-exact with the oracle"
    # unfold of the final codes and scales
    fp8, sc = g.rowmajor()
    q, owned, table = oracle.plan(w.dims, w.D, w.rank)
    E, H, W = w.dims[0]
    o8 = np.zeros((E, H, W), dtype=np.uint8)
    osc = np.zeros((E, 2, 3), dtype=np.float32)
    oracle.unpack(w.dims, ora["codes"].reshape(-1), ora["scale_inv"], table, [o8], [osc])
    assert np.array_equal(fp8[0].cpu().numpy().reshape(E, H, W), o8)
    assert np.array_equal(sc[0].cpu().numpy().reshape(E, 2, 3), osc)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("mode", MODES)
def test_ragged_every_slot(mode, layout):
    w = WL.ragged()
    _say("ragged: 40 matrices, D=8 rank 3, seed", w.seed, "mode", mode, "layout", layout)
    g = GpuWorkload(w, mode=mode, layout=layout)
    g.load_state()
    g.run_steps()
    slots = list(range(g.q))
    ora = oracle_slots(w, slots)
    rep = _check(g.tiles(slots), ora, "ragged")
    assert rep["exact"]
    # unfold into the ragged row-major weights
    fp8, sc = g.rowmajor()
    q, owned, table = oracle.plan(w.dims, w.D, w.rank)
    o8 = [None] * len(w.dims)
    osc = [None] * len(w.dims)
    for p in g.touched:
        E, H, W = w.dims[p]
        o8[p] = np.zeros((E, H, W), dtype=np.uint8)
        osc[p] = np.zeros((E, -(-H // 128), -(-W // 128)), dtype=np.float32)
    oracle.unpack(w.dims, ora["codes"].reshape(-1), ora["scale_inv"], table, o8, osc)
    for p in g.touched:
        assert np.array_equal(fp8[p].cpu().numpy().reshape(o8[p].shape), o8[p]), p
        assert np.array_equal(sc[p].cpu().numpy().reshape(osc[p].shape), osc[p]), p
    del g
    _free()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["dense_llm", "moe_experts", "large"])
def test_full_size_sampled(name, mode):
    w = WL.BY_NAME[name]()
    _say(name, "full size,", len(w.dims), "weights, D =", w.D, "rank", w.rank, "seed", w.seed,
         "mode", mode, "layout", BENCH_LAYOUT)
    g = GpuWorkload(w, mode=mode, layout=BENCH_LAYOUT)
    g.load_state()
    g.run_steps()
    slots = sample_slots(w)
    _say(name, "slots sampled:", len(slots), "of", g.q)
    ora = oracle_slots(w, slots)
    rep = _check(g.tiles(slots), ora, name)
    assert rep["exact"]
    if name == "large":
        # amax = 0 guard on the all-zero tiles of this workload
        zero = [k for k, s in enumerate(slots) if not ora["master"][k].any()]
        assert zero, "sample holds no all-zero tile"
        assert (ora["scale_inv"][zero] == 1.0).all()
        # row-major FP8 + scale grid, checked at the sampled tiles
        fp8, sc = g.rowmajor()
        torch.cuda.synchronize()
        for k, s in enumerate(slots):
            p, e, i, j, vr, vc = (int(x) for x in ora["table"][k])
            if p < 0:
                continue
            E, H, W = w.dims[p]
            block = fp8[p].view(E, H, W)[e, 128 * i:128 * i + vr, 128 * j:128 * j + vc]
            want = ora["codes"][k].reshape(128, 128)[:vr, :vc]
            assert np.array_equal(block.cpu().numpy(), want), (s, p, e, i, j)
            hb, wb = -(-H // 128), -(-W // 128)
            assert float(sc[p][(e * hb + i) * wb + j]) == float(ora["scale_inv"][k])
    del g
    _free()


def test_moe_full_size_every_slot():
    """The MoE expert shard (D = 32, rank 0: 21,504 tiles, 352M elements) at
    full size, in the launch configuration and state layout bench.py times,
    compared with the oracle on every slot -- master, m, v, tile-major codes
    and scale_inv, and the row-major FP8 weights and scale grid of every
    owned tile against the oracle's own unfold.  Compared in chunks of 2048
    slots so host memory stays bounded; midpoint cases are counted."""
    w = WL.moe()
    _say("moe_experts full size, every slot, mode fused_unpack, layout", BENCH_LAYOUT, "seed",
         w.seed)
    g = GpuWorkload(w, mode="fused_unpack", layout=BENCH_LAYOUT)
    g.load_state()
    g.run_steps()
    q, owned, table = oracle.plan(w.dims, w.D, w.rank)
    assert q == g.q == 21504 and owned == q
    ora_codes = np.empty((q, 16384), dtype=np.uint8)
    ora_scale = np.empty(q, dtype=np.float32)
    totals = {"codes_mismatch": 0, "codes_mismatch_near_midpoint": 0, "near_midpoint_elems": 0}
    exact = True
    chunk = 2048
    for s0 in range(0, q, chunk):
        slots = list(range(s0, min(q, s0 + chunk)))
        ora = oracle_slots(w, slots)
        rep = compare(g.tiles(slots), ora)
        assert rep["ok"], (s0, rep["fail"])
        exact &= rep["exact"]
        for k in totals:
            totals[k] += rep[k]
        ora_codes[s0:s0 + len(slots)] = ora["codes"]
        ora_scale[s0:s0 + len(slots)] = ora["scale_inv"]
        _say(f"moe slots {s0}..{s0 + len(slots) - 1}: exact={rep['exact']}")
        del ora
    _say("moe every slot:", q, "slots, bit-exact", exact, totals)
    assert exact
    # row-major output of the owned tiles (gate of experts 0..23): the
    # oracle's unfold of its own codes
    experts = int(table[owned - 1][1]) + 1
    E, H, W = w.dims[0]
    o8 = np.zeros((experts, H, W), dtype=np.uint8)
    osc = np.zeros((experts, -(-H // 128), -(-W // 128)), dtype=np.float32)
    oracle.unpack([(experts, H, W)], ora_codes.reshape(-1), ora_scale, table, [o8], [osc])
    fp8, sc = g.rowmajor()
    torch.cuda.synchronize()
    assert np.array_equal(fp8[0][:experts * H * W].cpu().numpy(), o8.reshape(-1))
    assert np.array_equal(sc[0][:osc.size].cpu().numpy(), osc.reshape(-1))
    del g
    _free()


def test_lone_rank_rowmajor_only_full_size():
    """The 2.01B-element workload (D = 1) as the bench steps it: the
    one-kernel step with no tile-major codes or scales, only the row-major
    FP8 weights and scale grids -- checked at the sampled tiles, with the
    master / moments, against the oracle."""
    w = WL.large()
    _say("large, row-major output only (lone rank), full size, layout", BENCH_LAYOUT)
    g = GpuWorkload(w, mode="fused_unpack", layout=BENCH_LAYOUT)
    g.tile_codes = False
    g.codes.fill_(0xAB)
    g.scale_inv.fill_(-7.0)
    g.load_state()
    g.run_steps()
    slots = sample_slots(w)
    ora = oracle_slots(w, slots)
    got = g.tiles(slots)
    assert (got["codes"] == 0xAB).all() and (got["scale_inv"] == -7.0).all()  # untouched
    for name in ("master", "m", "v"):
        assert np.array_equal(got[name].view(np.uint32), ora[name].view(np.uint32)), name
    fp8, sc = g.rowmajor()
    torch.cuda.synchronize()
    for k, s in enumerate(slots):
        p, e, i, j, vr, vc = (int(x) for x in ora["table"][k])
        E, H, W = w.dims[p]
        block = fp8[p].view(E, H, W)[e, 128 * i:128 * i + vr, 128 * j:128 * j + vc]
        assert np.array_equal(block.cpu().numpy(), ora["codes"][k].reshape(128, 128)[:vr, :vc]), s
        assert float(sc[p][(e * (H // 128) + i) * (W // 128) + j]) == float(ora["scale_inv"][k])
    del g, fp8, sc
    _free()


def _beyond_32bit():
    """The 2.01B-element recipe over 264 matrices of 4096x4096: 270,336
    tiles, 4.43B elements -- slot element offsets pass 2^31 (slot 131,072)
    and 2^32 (slot 262,144), and so do the byte offsets of the codes."""
    w = WL.large()
    w.name, w.config, w.seed = "beyond_32bit", 6, 6
    w.dims = [(1, 4096, 4096)] * 264
    w.description = "264 matrices of 4096x4096 (4.43B elements), D=1, t=1000"
    return w


_BIG = {}


# each route once; the one-kernel step in the interleaved layout, whose
# state offsets (slot * 50176 floats) pass 2^32 already at slot 85,599
@pytest.mark.parametrize("mode,layout", [("unfused", "separate"), ("fused", "separate"),
                                         ("fused_unpack", "interleaved")])
def test_offsets_beyond_32_bits(mode, layout):
    w = _beyond_32bit()
    _say("beyond 32-bit offsets:", w.description, "mode", mode, "layout", layout)
    g = GpuWorkload(w, mode=mode, layout=layout)
    assert g.q * 16384 > 2 ** 32
    g.load_state()
    g.run_steps()
    if "ora" not in _BIG:
        slots = sorted(set(sample_slots(w, n_random=40)) |
                       {131071, 131072, 262143, 262144, g.q - 1})
        _BIG["slots"], _BIG["ora"] = slots, oracle_slots(w, slots)
    slots, ora = _BIG["slots"], _BIG["ora"]
    rep = _check(g.tiles(slots), ora, "beyond_32bit " + mode)
    assert rep["exact"]
    fp8, sc = g.rowmajor()
    torch.cuda.synchronize()
    for k, s in enumerate(slots):
        p, e, i, j, vr, vc = (int(x) for x in ora["table"][k])
        E, H, W = w.dims[p]
        block = fp8[p].view(E, H, W)[e, 128 * i:128 * i + vr, 128 * j:128 * j + vc]
        assert np.array_equal(block.cpu().numpy(), ora["codes"][k].reshape(128, 128)[:vr, :vc]), s
        assert float(sc[p][(e * (H // 128) + i) * (W // 128) + j]) == float(ora["scale_inv"][k])
    del g, fp8, sc
    _free()


@pytest.mark.parametrize("mode", MODES)
def test_rank_decomposition_is_invariant(mode):
    """Every tile's result is independent of which rank owns it: the union
    of the D shards equals the single-rank run, bit for bit."""
    w1 = WL.ragged()
    w1.dims = w1.dims[:6]
    w1.D, w1.rank = 1, 0
    _say("rank invariance: 6 ragged matrices, D in {1, 3, 7}, mode", mode)
    ref = GpuWorkload(w1, mode=mode)
    ref.load_state()
    ref.run_steps()
    full = ref.tiles(list(range(ref.owned)))
    for D in (3, 7):
        parts = []
        for r in range(D):
            w = WL.ragged()
            w.dims, w.D, w.rank = w1.dims, D, r
            g = GpuWorkload(w, mode=mode)
            g.load_state()
            g.run_steps()
            if g.owned:
                parts.append(g.tiles(list(range(g.owned))))
            pad = list(range(g.owned, g.q))
            if pad:  # padding slots: zeros, scale 1, codes 0
                t = g.tiles(pad)
                assert not t["master"].any() and not t["codes"].any()
                assert (t["scale_inv"] == 1.0).all()
        for k in ("master", "m", "v", "codes", "scale_inv"):
            cat = np.concatenate([p[k] for p in parts])
            assert np.array_equal(cat.view(np.uint8), full[k].view(np.uint8)), (D, k)


def test_full_model_unfold_after_allgather():
    """Every rank steps its shard; the all-gather of the tile-major codes and
    scales is their concatenation in rank order, which puts every global tile
    at its global index -- so unpack_fp8 with the single-rank plan unfolds
    the whole model.  It must equal the single-rank run's row-major output."""
    dims = WL.ragged().dims[:7]
    D = 4
    _say("full-model unfold after all-gather: 7 ragged matrices, D =", D)
    codes, scales = [], []
    for r in range(D):
        w = WL.ragged()
        w.dims, w.D, w.rank = dims, D, r
        g = GpuWorkload(w, mode="fused_unpack")
        g.load_state()
        g.run_steps()
        codes.append(g.codes)
        scales.append(g.scale_inv)
    w1 = WL.ragged()
    w1.dims, w1.D, w1.rank = dims, 1, 0
    ref = GpuWorkload(w1, mode="fused_unpack")
    ref.load_state()
    ref.run_steps()
    T = ref.q
    gathered_codes = torch.cat(codes)[:T * 16384].contiguous()
    gathered_scales = torch.cat(scales)[:T].contiguous()
    fp8, sc = ref.alloc_rowmajor_out()
    bfz.unpack_fp8(ref.plan, gathered_codes, gathered_scales, fp8, sc)
    torch.cuda.synchronize()
    want8, wantsc = ref.rowmajor()
    for p in ref.touched:
        assert torch.equal(fp8[p], want8[p]), p
        assert torch.equal(sc[p], wantsc[p]), p


@pytest.mark.parametrize("seed", range(6))
def test_random_configurations(seed):
    """Random ragged weights, D, rank, hyper-parameters (weight decay 0 or
    not, large eps, step counters up to 10^6) and value scales, inputs drawn
    on the host with numpy; every slot of every entry point vs the oracle."""
    rng = np.random.default_rng(1000 + seed)
    dims = [(int(rng.integers(1, 3)), int(rng.integers(1, 400)), int(rng.integers(1, 400)))
            for _ in range(int(rng.integers(1, 5)))]
    D = int(rng.integers(1, 5))
    rank = int(rng.integers(0, D))
    hp = dict(lr=float(10 ** rng.uniform(-5, -1)), beta1=float(rng.choice([0.0, 0.5, 0.9])),
              beta2=float(rng.choice([0.9, 0.95, 0.999])), eps=float(10 ** rng.uniform(-10, -3)),
              weight_decay=float(rng.choice([0.0, 0.01, 0.3])))
    t = int(rng.choice([1, 2, 57, 10 ** 6]))
    pow2 = bool(seed % 2)
    _say("random config seed", 1000 + seed, "dims", dims, "D", D, "rank", rank, "hp", hp, "t", t,
         "pow2 scales", pow2)
    q, owned, table = oracle.plan(dims, D, rank)
    scale = float(10 ** rng.uniform(-4, 1))
    host = {k: [rng.normal(0, s, d).astype(np.float32) for d in dims]
            for k, s in (("p", scale), ("g", scale * 1e-2), ("m", scale * 1e-3))}
    host["v"] = [np.square(rng.normal(0, scale * 1e-2, d)).astype(np.float32) for d in dims]
    ora_state = {k: oracle.pack(dims, host[k], table) for k in ("p", "g", "m", "v")}
    codes_o, scale_o, near_o = oracle.step(ora_state["p"], ora_state["g"], ora_state["m"],
                                           ora_state["v"], oracle.hparams(step=t, **hp), pow2=pow2)
    plan = bfz.Plan(dims, D, rank)
    dev = {k: [torch.from_numpy(x.reshape(-1)).cuda() for x in host[k]] for k in host}
    for route in ("unfused", "fused", "fused_unpack"):
        st = {}
        for k in ("p", "m", "v"):
            st[k] = torch.empty(q * 16384, dtype=torch.float32, device="cuda")
            bfz.pack_shard(plan, dev[k], st[k])
        codes = torch.empty(q * 16384, dtype=torch.uint8, device="cuda")
        sc = torch.empty(q, dtype=torch.float32, device="cuda")
        h = bfz.AdamW(step=t, **hp)
        if route == "unfused":
            gt = torch.empty(q * 16384, dtype=torch.float32, device="cuda")
            bfz.pack_shard(plan, dev["g"], gt)
            bfz.adamw_fp8_step(st["p"], gt, st["m"], st["v"], codes, sc, h, scale_pow2=pow2)
        elif route == "fused":
            bfz.fold_adamw_fp8_step(plan, dev["g"], st["p"], st["m"], st["v"], codes, sc, h,
                                    scale_pow2=pow2)
        else:
            d8 = [torch.zeros(int(np.prod(d)), dtype=torch.uint8, device="cuda") for d in dims]
            dsc = [torch.zeros(d[0] * -(-d[1] // 128) * -(-d[2] // 128), dtype=torch.float32,
                               device="cuda") for d in dims]
            bfz.fold_adamw_fp8_step_unpack(plan, dev["g"], st["p"], st["m"], st["v"], codes, sc,
                                           d8, dsc, h, scale_pow2=pow2)
        torch.cuda.synchronize()
        gpu = dict(master=st["p"].cpu().numpy(), m=st["m"].cpu().numpy(), v=st["v"].cpu().numpy(),
                   codes=codes.cpu().numpy(), scale_inv=sc.cpu().numpy())
        ora = dict(master=ora_state["p"], m=ora_state["m"], v=ora_state["v"], codes=codes_o,
                   scale_inv=scale_o, near=near_o)
        rep = _check(gpu, ora, f"random seed {1000 + seed} {route}")
        assert rep["exact"]
        if route == "fused_unpack":
            o8 = [np.zeros(d, dtype=np.uint8) for d in dims]
            osc = [np.zeros((d[0], -(-d[1] // 128), -(-d[2] // 128)), dtype=np.float32) for d in dims]
            oracle.unpack(dims, codes_o, scale_o, table, o8, osc)
            for k in range(len(dims)):
                assert np.array_equal(d8[k].cpu().numpy(), o8[k].reshape(-1)), k
                assert np.array_equal(dsc[k].cpu().numpy(), osc[k].reshape(-1)), k


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("pow2", [False, True])
def test_many_weights_several_segments(pow2, layout):
    """A rank that owns 70+ small ragged weights, starting and ending
    mid-weight: its slots span several launch segments (at most 64 weights
    each) in every route -- tile-major step, fused fold, one-kernel step
    and, with power-of-two scales, the step that also writes W^T -- each
    checked on every slot and every row-major output against the oracle."""
    rng = np.random.default_rng(2000 + int(pow2))
    dims = [(int(rng.integers(1, 3)), int(rng.integers(1, 260)), int(rng.integers(1, 260)))
            for _ in range(250)]
    D, rank = 3, 1
    q, owned, table = oracle.plan(dims, D, rank)
    touched = sorted(set(int(p) for p in table[:owned, 0]))
    assert len(touched) > 64 and owned > 0
    assert tuple(table[0][1:4]) != (0, 0, 0)                         # starts inside a weight
    assert oracle.plan(dims, D, rank + 1)[2][0][0] == table[owned - 1][0]  # ends inside one
    _say("many weights: 250 ragged, D", D, "rank", rank, "owns", owned, "tiles of", len(touched),
         "weights, pow2", pow2, "layout", layout)
    host = {k: [rng.normal(0, s, d).astype(np.float32) for d in dims]
            for k, s in (("p", 0.02), ("g", 1e-3), ("m", 1e-4))}
    host["v"] = [np.square(rng.normal(0, 1e-3, d)).astype(np.float32) for d in dims]
    ora = {k: oracle.pack(dims, host[k], table) for k in ("p", "g", "m", "v")}
    hp = dict(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    codes_o, scale_o, near_o = oracle.step(ora["p"], ora["g"], ora["m"], ora["v"],
                                           oracle.hparams(step=3, **hp), pow2=pow2)
    o8 = [np.zeros(d, dtype=np.uint8) for d in dims]
    osc = [np.zeros((d[0], -(-d[1] // 128), -(-d[2] // 128)), dtype=np.float32) for d in dims]
    oracle.unpack(dims, codes_o, scale_o, table, o8, osc)
    if pow2:
        ot = [np.zeros((d[0], d[2], d[1]), dtype=np.uint8) for d in dims]
        ots = [np.zeros((d[0], d[2], -(-d[1] // 128)), dtype=np.float32) for d in dims]
        oracle.transpose_pow2(dims, codes_o, scale_o, table, ot, ots)
    plan = bfz.Plan(dims, D, rank)
    dev = {k: [torch.from_numpy(x.reshape(-1)).cuda() for x in host[k]] for k in host}
    routes = ["unfused", "fused", "fused_unpack"] + (["fused_unpack_t"] if pow2 else [])
    for route in routes:
        st = {}
        if layout == "interleaved":  # segments start at slot0 * 49152 floats of one buffer
            state = torch.empty((q, 3, 16384), dtype=torch.float32, device="cuda")
            st = {"p": state[:, 0], "m": state[:, 1], "v": state[:, 2]}
        for k in ("p", "m", "v"):
            if layout == "separate":
                st[k] = torch.empty(q * 16384, dtype=torch.float32, device="cuda")
            bfz.pack_shard(plan, dev[k], st[k])
        codes = torch.empty(q * 16384, dtype=torch.uint8, device="cuda")
        sc = torch.empty(q, dtype=torch.float32, device="cuda")
        h = bfz.AdamW(step=3, **hp)
        d8 = [torch.zeros(int(np.prod(d)), dtype=torch.uint8, device="cuda") for d in dims]
        dsc = [torch.zeros(osc[k].size, dtype=torch.float32, device="cuda") for k in range(len(dims))]
        if route == "unfused":
            gt = torch.empty(q * 16384, dtype=torch.float32, device="cuda")
            bfz.pack_shard(plan, dev["g"], gt)
            bfz.adamw_fp8_step(st["p"], gt, st["m"], st["v"], codes, sc, h, scale_pow2=pow2)
            bfz.unpack_fp8(plan, codes, sc, d8, dsc)
        elif route == "fused":
            bfz.fold_adamw_fp8_step(plan, dev["g"], st["p"], st["m"], st["v"], codes, sc, h,
                                    scale_pow2=pow2)
            bfz.unpack_fp8(plan, codes, sc, d8, dsc)
        elif route == "fused_unpack":
            bfz.fold_adamw_fp8_step_unpack(plan, dev["g"], st["p"], st["m"], st["v"], codes, sc,
                                           d8, dsc, h, scale_pow2=pow2)
        else:
            dt = [torch.zeros(int(np.prod(d)), dtype=torch.uint8, device="cuda") for d in dims]
            dts = [torch.zeros(ots[k].size, dtype=torch.float32, device="cuda")
                   for k in range(len(dims))]
            bfz.fold_adamw_fp8_step_unpack_t(plan, dev["g"], st["p"], st["m"], st["v"], codes, sc,
                                             d8, dsc, dt, dts, h)
        torch.cuda.synchronize()
        gpu = dict(master=st["p"].cpu().numpy().reshape(-1), m=st["m"].cpu().numpy().reshape(-1),
                   v=st["v"].cpu().numpy().reshape(-1), codes=codes.cpu().numpy(),
                   scale_inv=sc.cpu().numpy())
        rep = _check(gpu, dict(master=ora["p"], m=ora["m"], v=ora["v"], codes=codes_o,
                               scale_inv=scale_o, near=near_o), f"many weights {route} {layout}")
        assert rep["exact"]
        for k in range(len(dims)):
            assert np.array_equal(d8[k].cpu().numpy(), o8[k].reshape(-1)), (route, k)
            assert np.array_equal(dsc[k].cpu().numpy(), osc[k].reshape(-1)), (route, k)
            if route == "fused_unpack_t":
                assert np.array_equal(dt[k].cpu().numpy(), ot[k].reshape(-1)), (route, k)
                assert np.array_equal(dts[k].cpu().numpy(), ots[k].reshape(-1)), (route, k)


def test_amax_at_every_position():
    """16384 tiles; tile k has its largest |value| at element k (sign
    alternating).  lr = 0 leaves the master unchanged, so the scale must be
    1/448 in every tile, the code there 0x7E / 0xFE, and every code must
    match the oracle on a sample of tiles."""
    n = 16384
    _say("amax at every position:", n, "tiles, seed 11")
    rng = np.random.default_rng(11)
    host = rng.uniform(-0.5, 0.5, (n, 16384)).astype(np.float32)
    k = np.arange(n)
    host[k, k] = np.where(k % 2 == 0, 1.0, -1.0).astype(np.float32)
    dev = torch.from_numpy(host).cuda().view(-1)
    z = torch.zeros_like(dev)
    m, v = z.clone(), z.clone()
    codes = torch.empty(dev.numel(), dtype=torch.uint8, device="cuda")
    scale = torch.empty(n, dtype=torch.float32, device="cuda")
    hp = bfz.AdamW(lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    bfz.adamw_fp8_step(dev, z, m, v, codes, scale, hp)
    torch.cuda.synchronize()
    s = scale.cpu().numpy()
    assert (s == np.float32(1.0) / np.float32(448.0)).all()
    c = codes.view(n, 16384).cpu().numpy()
    assert (c[k, k] == np.where(k % 2 == 0, 0x7E, 0xFE)).all()
    assert np.array_equal(dev.view(n, 16384).cpu().numpy(), host)
    sample = rng.choice(n, 64, replace=False)
    oc, osc, _ = oracle.quant_tiles(np.ascontiguousarray(host[sample]).reshape(-1))
    assert np.array_equal(c[sample].reshape(-1), oc)
    del dev, z, m, v, codes
    _free()


def test_deterministic_and_empty():
    w = WL.tiny()
    _say("determinism + n_tiles=0, tiny")
    outs = []
    for _ in range(2):
        g = GpuWorkload(w)
        g.load_state()
        g.run_steps()
        outs.append(g.tiles(list(range(g.q))))
    for k in outs[0]:
        assert np.array_equal(outs[0][k].view(np.uint8), outs[1][k].view(np.uint8)), k
    before = g.codes.clone()
    bfz.adamw_fp8_step(g.master, g.grad, g.m, g.v, g.codes, g.scale_inv,
                       bfz.AdamW(step=4, **WL.HP), n_tiles=0)
    torch.cuda.synchronize()
    assert torch.equal(before, g.codes)


@pytest.mark.parametrize("off", [1, 2, 3])
def test_fused_routes_equal_unfused_on_misaligned_buffers(off):
    """Gradients that start `off` floats into their buffer (no 16-byte
    vector path) and FP8 destinations that start 1 byte in (no 32-bit
    stores) give the same bits through all routes, and without the
    tile-major copy.  The reference route steps the oracle's fold of the
    gradients, so it shares no row-major loader with the routes checked."""
    dims = [(1, 300, 260), (2, 129, 516), (1, 128, 128), (1, 131, 387)]
    _say("fused vs oracle fold + step, gradients offset by", off, "floats, seed", 20 + off)
    rng = np.random.default_rng(20 + off)
    plan = bfz.Plan(dims, 2, 1)
    q = plan.shard_tiles
    n = q * 16384
    state0 = [torch.from_numpy(rng.normal(0, s, n).astype(np.float32)).cuda()
              for s in (0.02, 1e-4, 1e-7)]
    for x in state0:  # padding slots hold zero state
        x.view(q, 16384)[plan.owned_tiles:] = 0
    state0[2].abs_()
    grads, host_grads = [], []
    for d in dims:
        h = rng.normal(0, 1e-3, d).astype(np.float32)
        raw = torch.zeros(h.size + 4, dtype=torch.float32, device="cuda")
        raw[off:off + h.size] = torch.from_numpy(h.reshape(-1)).cuda()
        grads.append(raw[off:off + h.size])
        host_grads.append(h)
    _, _, table = oracle.plan(dims, 2, 1)
    folded = torch.from_numpy(oracle.pack(dims, host_grads, table)).cuda()
    hb = [(d[0], -(-d[1] // 128), -(-d[2] // 128)) for d in dims]
    outs = []
    for route in ("unfused", "fused", "fused_unpack", "rowmajor_only"):
        p, m, v = (x.clone() for x in state0)
        codes = torch.zeros(n, dtype=torch.uint8, device="cuda")
        sc = torch.zeros(q, dtype=torch.float32, device="cuda")
        raw8 = [torch.zeros(int(np.prod(d)) + 1, dtype=torch.uint8, device="cuda") for d in dims]
        d8 = [r[1:] for r in raw8]
        dsc = [torch.zeros(int(np.prod(h)), dtype=torch.float32, device="cuda") for h in hb]
        hp = bfz.AdamW(step=5, **WL.HP)
        if route == "unfused":
            bfz.adamw_fp8_step(p, folded, m, v, codes, sc, hp)
            bfz.unpack_fp8(plan, codes, sc, d8, dsc)
        elif route == "fused":
            bfz.fold_adamw_fp8_step(plan, grads, p, m, v, codes, sc, hp)
            bfz.unpack_fp8(plan, codes, sc, d8, dsc)
        elif route == "fused_unpack":
            bfz.fold_adamw_fp8_step_unpack(plan, grads, p, m, v, codes, sc, d8, dsc, hp)
        else:
            bfz.fold_adamw_fp8_step_unpack(plan, grads, p, m, v, None, None, d8, dsc, hp)
        torch.cuda.synchronize()
        outs.append([x.cpu().numpy() for x in [p, m, v, codes, sc] + d8 + dsc])
    for r in range(1, 4):
        for k, (a, b) in enumerate(zip(outs[0], outs[r])):
            if r == 3 and k in (3, 4):
                assert not b.any()  # no tile-major copy requested
                continue
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (r, k)


def test_misaligned_pointer_is_rejected():
    _say("alignment errors")
    x = torch.zeros(2 * 16384 + 4, dtype=torch.float32, device="cuda")
    c = torch.zeros(2 * 16384 + 16, dtype=torch.uint8, device="cuda")
    s = torch.zeros(2, dtype=torch.float32, device="cuda")
    off = x[1:1 + 16384]
    with pytest.raises(bfz.BfzError) as e:
        bfz.adamw_fp8_step(off, off, off, off, c[:16384], s, bfz.AdamW(step=1, **WL.HP))
    assert e.value.code == bfz.BFZ_EALIGN


@pytest.mark.parametrize("pow2", [False, True])
def test_subnormal_masters_and_edge_amax(pow2):
    """Host-forced cases, bit-exact against the oracle through all routes:
    the tile amax in the last valid cell next to the padding of edge tiles;
    a tile of subnormal masters with zero gradient and state, which stays
    subnormal, so amax / 448 underflows and the 2^-149 floor applies; a tile
    where subnormal gradients meet subnormal masters; a normal expert."""
    tiny = 2.0 ** -149
    dims = [(1, 130, 200), (2, 128, 256)]
    _say("subnormal masters and pad-adjacent amax, pow2", pow2)
    rng = np.random.default_rng(55)
    w0 = rng.normal(0, 0.02, (1, 130, 200))
    w0[0, 129, 199], w0[0, 127, 199], w0[0, 129, 127] = 0.5, -0.4, 0.3
    g0 = rng.normal(0, 1e-3, (1, 130, 200))
    w1 = rng.normal(0, 0.02, (2, 128, 256))
    g1 = rng.normal(0, 1e-3, (2, 128, 256))
    w1[0, :, :128] = rng.integers(-200, 201, (128, 128)) * tiny      # underflowing tile
    g1[0, :, :128] = 0.0
    w1[0, :, 128:] = rng.integers(-2 ** 20, 2 ** 20, (128, 128)) * tiny
    g1[0, :, 128:] = rng.integers(-1000, 1001, (128, 128)) * tiny
    masters = [w0.astype(np.float32), w1.astype(np.float32)]
    grads = [g0.astype(np.float32), g1.astype(np.float32)]
    assert np.abs(masters[1][0, :, :128]).max() <= np.float32(224 * tiny)
    q, owned, table = oracle.plan(dims, 1, 0)
    p0 = oracle.pack(dims, masters, table)
    gt = oracle.pack(dims, grads, table)
    n = q * 16384
    steps = (1, 2)
    op, om, ov = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in steps:
        ocodes, oscale, _ = oracle.step(op, gt, om, ov, oracle.hparams(step=t, **WL.HP), 1e-6, pow2)
    assert (oscale[:q] > 0).all()
    odst8 = [np.zeros(d, np.uint8) for d in dims]
    odsc = [np.zeros((E, -(-H // 128), -(-W // 128)), np.float32) for E, H, W in dims]
    oracle.unpack(dims, ocodes, oscale, table, odst8, odsc)
    plan = bfz.Plan(dims, 1, 0)
    g_dev = [torch.from_numpy(g.reshape(-1)).cuda() for g in grads]
    gt_dev = torch.from_numpy(gt).cuda()
    for route in ("unfused", "fused", "fused_unpack"):
        p = torch.from_numpy(p0).cuda()
        m = torch.zeros(n, dtype=torch.float32, device="cuda")
        v = torch.zeros(n, dtype=torch.float32, device="cuda")
        codes = torch.zeros(n, dtype=torch.uint8, device="cuda")
        sc = torch.zeros(q, dtype=torch.float32, device="cuda")
        d8 = [torch.zeros(int(np.prod(d)), dtype=torch.uint8, device="cuda") for d in dims]
        dsc = [torch.zeros(x.size, dtype=torch.float32, device="cuda") for x in odsc]
        for t in steps:
            hp = bfz.AdamW(step=t, **WL.HP)
            if route == "unfused":
                bfz.adamw_fp8_step(p, gt_dev, m, v, codes, sc, hp, scale_pow2=pow2)
            elif route == "fused":
                bfz.fold_adamw_fp8_step(plan, g_dev, p, m, v, codes, sc, hp, scale_pow2=pow2)
            else:
                bfz.fold_adamw_fp8_step_unpack(plan, g_dev, p, m, v, codes, sc, d8, dsc, hp,
                                               scale_pow2=pow2)
        if route != "fused_unpack":
            bfz.unpack_fp8(plan, codes, sc, d8, dsc)
        torch.cuda.synchronize()
        for name, got, want in (("master", p, op), ("m", m, om), ("v", v, ov), ("codes", codes, ocodes),
                                ("scale_inv", sc, oscale)):
            g_np = got.cpu().numpy()
            assert np.array_equal(g_np.view(np.uint8), want.view(np.uint8)), (route, name)
        for k in range(len(dims)):
            assert np.array_equal(d8[k].cpu().numpy(), odst8[k].reshape(-1)), (route, "fp8", k)
            assert np.array_equal(dsc[k].cpu().numpy(), odsc[k].reshape(-1)), (route, "grid", k)


@pytest.mark.parametrize("mode", MODES)
def test_runs_on_the_callers_stream(mode):
    """Every call is enqueued on the caller's current stream: a side stream
    that waits for the set-up, takes all steps and is then waited for gives
    bit for bit the default stream's result.  A call that went to another
    stream would race with the set-up or the read-back."""
    w = WL.ragged()
    w.dims = w.dims[:12]
    _say("side stream vs default stream, 12 ragged matrices, mode", mode)
    outs = []
    for side in (False, True):
        g = GpuWorkload(w, mode=mode)
        g.load_state()
        if side:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for t in w.steps:
                    g.draw_grads(t)
                    g.apply(t)
                fp8, sc = g.rowmajor()
            torch.cuda.current_stream().wait_stream(s)
        else:
            g.run_steps()
            fp8, sc = g.rowmajor()
        torch.cuda.synchronize()
        tiles = g.tiles(list(range(g.q)))
        outs.append((tiles, [x.cpu().numpy() if x is not None else None for x in fp8 + sc]))
        del g
        _free()
    (ta, ra), (tb, rb) = outs
    for k in ta:
        assert np.array_equal(ta[k].view(np.uint8), tb[k].view(np.uint8)), k
    for a, b in zip(ra, rb):
        assert (a is None and b is None) or np.array_equal(a, b)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_long_trajectory_every_slot(layout):
    """40 consecutive steps (t = 1 .. 40, fresh gradients each step) on
    small ragged weights, D = 2 rank 1, through the one-kernel step: every
    slot equals the oracle's own 40-step trajectory bit for bit, and so do
    the row-major outputs of the last step."""
    w = WL.ragged()
    w.dims = [(1, 300, 410), (2, 130, 257), (1, 77, 1000)]
    w.D, w.rank = 2, 1
    w.steps = list(range(1, 41))
    _say("40-step trajectory: 3 small ragged weights, D = 2 rank 1, layout", layout)
    g = GpuWorkload(w, mode="fused_unpack", layout=layout)
    g.load_state()
    g.run_steps()
    slots = list(range(g.q))
    ora = oracle_slots(w, slots)
    rep = _check(g.tiles(slots), ora, f"40 steps, {layout}")
    assert rep["exact"]
    fp8, sc = g.rowmajor()
    torch.cuda.synchronize()
    q, owned, table = oracle.plan(w.dims, w.D, w.rank)
    o8 = [np.zeros(d, dtype=np.uint8) for d in w.dims]
    osc = [np.zeros((d[0], -(-d[1] // 128), -(-d[2] // 128)), dtype=np.float32) for d in w.dims]
    oracle.unpack(w.dims, ora["codes"].reshape(-1), ora["scale_inv"], table, o8, osc)
    for k in range(owned):
        p, e, i, j, vr, vc = (int(x) for x in table[k])
        E, H, W = w.dims[p]
        got = fp8[p].view(E, H, W)[e, 128 * i:128 * i + vr, 128 * j:128 * j + vc].cpu().numpy()
        assert np.array_equal(got, o8[p][e, 128 * i:128 * i + vr, 128 * j:128 * j + vc]), k
        assert float(sc[p].view(osc[p].shape)[e, i, j]) == float(osc[p][e, i, j]), k
