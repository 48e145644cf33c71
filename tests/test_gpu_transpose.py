"""GPU parity of the power-of-two step and of the exponent-edit transpose
(bfz_transpose_pow2) against the oracle (needs an MI355X).  Byte results
must be bit-exact."""
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
    print("[gpu-transpose]", *a, flush=True)
    sys.stdout.flush()


def _outputs(dims, device):
    dt = [torch.full((E * W * H,), 0xAA, dtype=torch.uint8, device=device) for E, H, W in dims]
    ds = [torch.full((E * W * -(-H // 128),), -1.0, dtype=torch.float32, device=device)
          for E, H, W in dims]
    return dt, ds


def _oracle_outputs(dims):
    dt = [np.full((E, W, H), 0xAA, dtype=np.uint8) for E, H, W in dims]
    ds = [np.full((E, W, -(-H // 128)), -1.0, dtype=np.float32) for E, H, W in dims]
    return dt, ds


CASES = [
    ([(1, 256, 384)], 1, 0),
    ([(2, 300, 129), (1, 77, 513), (1, 1, 1)], 1, 0),
    ([(3, 129, 130), (1, 128, 1000)], 3, 1),
    ([(1, 640, 48)] * 140, 2, 1),  # rank owns 70 weights: several launch segments
    # tall weights: ownership cut inside tile columns, tile-row counts that
    # are not multiples of 4
    ([(1, 1100, 300), (2, 700, 520)], 3, 1),
    ([(1, 2000, 130), (1, 129, 4000)], 5, 2),
    ([(1, 1024, 256)], 2, 1),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_transpose_random_codes(case):
    """Random codes (NaN patterns excluded) on random power-of-two scales,
    including the 2^-149 floor, with zero columns mixed in."""
    dims, D, rank = CASES[case]
    _say("random codes case", case, "D", D, "rank", rank, "weights", len(dims))
    rng = np.random.default_rng(40 + case)
    q, owned, table = oracle.plan(dims, D, rank)
    codes = rng.integers(0, 256, q * 16384).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    codes.reshape(q, 128, 128)[:, :, ::7] = 0              # all-zero columns
    codes.reshape(q, 128, 128)[:, :, 3::11] &= 0x87        # small magnitudes, subnormals
    T = rng.integers(-149, 100, q)
    T[: min(q, 3)] = [-149, -145, -140][: min(q, 3)]
    scale = np.ldexp(1.0, T).astype(np.float32)
    odt, ods = _oracle_outputs(dims)
    oracle.transpose_pow2(dims, codes, scale, table, odt, ods)
    plan = bfz.Plan(dims, D, rank)
    dt, ds = _outputs(dims, "cuda")
    bfz.transpose_pow2(plan, torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(), dt, ds)
    torch.cuda.synchronize()
    for p in range(len(dims)):
        assert np.array_equal(dt[p].cpu().numpy(), odt[p].reshape(-1)), p
        assert np.array_equal(ds[p].cpu().numpy(), ods[p].reshape(-1)), p


@pytest.mark.parametrize("mode", GpuWorkload.MODES)
def test_pow2_step_then_transpose(mode):
    """The flow: a power-of-two step of the ragged workload (every slot vs
    the oracle), then the transposed copy of its codes."""
    w = WL.ragged()
    w.dims = w.dims[:10]
    _say("pow2 step + transpose: 10 ragged matrices, D=8 rank 3, mode", mode)
    g = GpuWorkload(w, mode=mode, pow2=True)
    g.load_state()
    g.run_steps()
    slots = list(range(g.q))
    ora = oracle_slots(w, slots, pow2=True)
    rep = compare(g.tiles(slots), ora)
    _say({k: v for k, v in rep.items() if k != "fail"})
    assert rep["ok"] and rep["exact"], rep["fail"]
    sc = ora["scale_inv"]
    assert (np.frexp(sc)[0] == 0.5).all()
    q, owned, table = oracle.plan(w.dims, w.D, w.rank)
    odt, ods = _oracle_outputs(w.dims)
    oracle.transpose_pow2(w.dims, ora["codes"].reshape(-1), sc, table, odt, ods)
    dt, ds = _outputs(w.dims, "cuda")
    bfz.transpose_pow2(g.plan, g.codes, g.scale_inv, dt, ds)
    torch.cuda.synchronize()
    for p in g.touched:
        assert np.array_equal(dt[p].cpu().numpy(), odt[p].reshape(-1)), p
        assert np.array_equal(ds[p].cpu().numpy(), ods[p].reshape(-1)), p


def test_transpose_quantized_weights():
    """Codes of power-of-two-quantized Gaussian weights on full, 16-byte
    aligned tiles -- mostly normal codes, where whole words are moved at
    once -- with a sprinkling of values small enough to give subnormal
    codes, and zero columns, so both routes meet inside one wave."""
    dims = [(2, 512, 384), (1, 1024, 640), (1, 256, 4096)]
    _say("quantized Gaussian weights", dims)
    rng = np.random.default_rng(77)
    ws = []
    for E, H, W in dims:
        x = rng.normal(0, 1, (E, H, W)) * 10.0 ** rng.uniform(-1, 0.5, (E, 1, W))
        amax = np.abs(x).max()
        tiny = rng.random((E, H, W)) < 2e-4
        x[tiny] = amax * 2.0 ** -13 * np.sign(rng.normal(size=int(tiny.sum())))
        x[:, :, ::37] = 0.0
        ws.append(x.astype(np.float32))
    q, owned, table = oracle.plan(dims, 1, 0)
    codes, scale, _ = oracle.quant_tiles(oracle.pack(dims, ws, table), pow2=True)
    mags = codes & 0x7F
    assert ((mags > 0) & (mags < 8)).sum() > 100 and (mags >= 8).mean() > 0.5
    odt, ods = _oracle_outputs(dims)
    oracle.transpose_pow2(dims, codes, scale, table, odt, ods)
    plan = bfz.Plan(dims, 1, 0)
    dt, ds = _outputs(dims, "cuda")
    bfz.transpose_pow2(plan, torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(), dt, ds)
    torch.cuda.synchronize()
    for p in range(len(dims)):
        assert np.array_equal(dt[p].cpu().numpy(), odt[p].reshape(-1)), p
        assert np.array_equal(ds[p].cpu().numpy(), ods[p].reshape(-1)), p


@pytest.mark.parametrize("tile_codes,layout", [(True, "separate"), (False, "separate"),
                                               (True, "interleaved")])
def test_fused_step_with_transposed_copy(tile_codes, layout):
    """fold_adamw_fp8_step_unpack_t over the steps of ten ragged matrices:
    master, moments, codes and scales, the row-major FP8 weights and the
    transposed copy all equal the oracle's power-of-two step followed by its
    unfold and its transposed copy, bit for bit (without the tile-major copy
    when tile_codes is False: those buffers stay untouched)."""
    w = WL.ragged()
    w.dims = w.dims[:10]
    _say("fused step + transposed copy: 10 ragged matrices, D=8 rank 3, tile codes", tile_codes,
         "layout", layout)
    g = GpuWorkload(w, mode="fused_unpack", pow2=True, transposed=True, layout=layout)
    g.tile_codes = tile_codes
    g.codes.fill_(0xAB)
    g.scale_inv.fill_(-7.0)
    g.load_state()
    g.run_steps()
    slots = list(range(g.q))
    ora = oracle_slots(w, slots, pow2=True)
    got = g.tiles(slots)
    for name in ("master", "m", "v"):
        assert np.array_equal(got[name].view(np.uint32), ora[name].view(np.uint32)), name
    if tile_codes:
        assert np.array_equal(got["codes"], ora["codes"]) and np.array_equal(got["scale_inv"], ora["scale_inv"])
    else:
        assert (got["codes"] == 0xAB).all() and (got["scale_inv"] == -7.0).all()
    q, owned, table = oracle.plan(w.dims, w.D, w.rank)
    o8 = [np.zeros((E, H, W), np.uint8) for E, H, W in w.dims]
    osc = [np.zeros((E, -(-H // 128), -(-W // 128)), np.float32) for E, H, W in w.dims]
    oracle.unpack(w.dims, ora["codes"].reshape(-1), ora["scale_inv"], table, o8, osc)
    odt, ods = _oracle_outputs(w.dims)
    oracle.transpose_pow2(w.dims, ora["codes"].reshape(-1), ora["scale_inv"], table, odt, ods)
    torch.cuda.synchronize()
    for p in g.touched:
        E, H, W = w.dims[p]
        rows = table[:owned][table[:owned, 0] == p]
        # only the rank's own tiles are written: compare those blocks
        fp8 = g.out_fp8[p].view(E, H, W).cpu().numpy()
        wt = g.out_t[p].view(E, W, H).cpu().numpy()
        wts = g.out_t_scale[p].view(E, W, -(-H // 128)).cpu().numpy()
        sc = g.out_scale[p].view(E, -(-H // 128), -(-W // 128)).cpu().numpy()
        for _, e, i, j, vr, vc in rows:
            assert np.array_equal(fp8[e, 128 * i:128 * i + vr, 128 * j:128 * j + vc],
                                  o8[p][e, 128 * i:128 * i + vr, 128 * j:128 * j + vc]), (p, e, i, j)
            assert sc[e, i, j] == osc[p][e, i, j]
            assert np.array_equal(wt[e, 128 * j:128 * j + vc, 128 * i:128 * i + vr],
                                  odt[p][e, 128 * j:128 * j + vc, 128 * i:128 * i + vr]), (p, e, i, j)
            assert np.array_equal(wts[e, 128 * j:128 * j + vc, i], ods[p][e, 128 * j:128 * j + vc, i])
    del g


def test_fused_transposed_copy_full_size_sampled():
    """The dense-LLM shard (all 11 steps) through fold_adamw_fp8_step_unpack_t,
    as bench.py --path fused_unpack_t times it: sampled tiles against the
    oracle -- state, codes, scales, row-major FP8 and the W^T block with its
    group scales (the oracle's transposed copy of that tile alone)."""
    w = WL.dense_llm()
    _say("dense_llm full size, fused step + transposed copy, pow2, interleaved state")
    g = GpuWorkload(w, mode="fused_unpack", pow2=True, transposed=True, layout="interleaved")
    g.load_state()
    g.run_steps()
    slots = sample_slots(w, n_random=48)
    ora = oracle_slots(w, slots, pow2=True)
    rep = compare(g.tiles(slots), ora)
    _say({k: v for k, v in rep.items() if k != "fail"})
    assert rep["ok"] and rep["exact"], rep["fail"]
    torch.cuda.synchronize()
    for k, s in enumerate(slots):
        p, e, i, j, vr, vc = (int(x) for x in ora["table"][k])
        if p < 0:
            continue
        E, H, W = w.dims[p]
        hb = -(-H // 128)
        block = g.out_fp8[p].view(E, H, W)[e, 128 * i:128 * i + vr, 128 * j:128 * j + vc]
        assert np.array_equal(block.cpu().numpy(), ora["codes"][k].reshape(128, 128)[:vr, :vc]), s
        one_dt = [np.zeros((1, vc, vr), np.uint8)]
        one_ds = [np.zeros((1, vc, 1), np.float32)]
        oracle.transpose_pow2([(1, vr, vc)], np.ascontiguousarray(ora["codes"][k].reshape(-1)),
                              np.array([ora["scale_inv"][k]], np.float32),
                              np.array([[0, 0, 0, 0, vr, vc]], np.int64), one_dt, one_ds)
        wt = g.out_t[p].view(E, W, H)[e, 128 * j:128 * j + vc, 128 * i:128 * i + vr]
        wts = g.out_t_scale[p].view(E, W, hb)[e, 128 * j:128 * j + vc, i]
        assert np.array_equal(wt.cpu().numpy(), one_dt[0][0]), s
        assert np.array_equal(wts.cpu().numpy(), one_ds[0][0, :, 0]), s
    del g
