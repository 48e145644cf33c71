"""GPU parity of fold (pack_shard), unfold (unpack_fp8) and the E4M3
rounding against the oracle (needs an MI355X).

Byte work must be bit-exact.  Inputs are seeded numpy draws (random floats
for fold, random bytes for unfold) over shapes that cover aligned weights
(vector path), widths that are not multiples of 4 or 16 (scalar / byte
paths), several experts, several weights per launch and more ranks than
tiles (padding slots)."""
import sys

import numpy as np
import pytest
import torch

import blockwise_fp8_zero_amd as bfz
import oracle

pytestmark = pytest.mark.gpu

CASES = [
    ([(1, 256, 384)], 1, 0),
    ([(1, 129, 300), (2, 200, 257), (1, 1, 1), (3, 128, 128)], 1, 0),
    ([(1, 129, 300), (2, 200, 257), (1, 1, 1), (3, 128, 128)], 3, 1),
    ([(2, 383, 130), (1, 77, 1029), (1, 640, 16)], 4, 3),
    ([(1, 200, 130)], 3, 2),            # more ranks than tiles: rank 2 owns nothing
    ([(1, 130, 131)] * 140, 2, 1),      # rank owns 70 weights: several launch segments
]


def _say(*a):
    print("[gpu-layout]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("case", range(len(CASES)))
def test_pack_matches_oracle(case):
    dims, D, rank = CASES[case]
    _say("pack case", case, "D", D, "rank", rank, "weights", len(dims))
    rng = np.random.default_rng(case)
    hosts = [rng.normal(0, 1, d).astype(np.float32) for d in dims]
    q, owned, table = oracle.plan(dims, D, rank)
    want = oracle.pack(dims, hosts, table)
    plan = bfz.Plan(dims, D, rank)
    assert np.array_equal(plan.table(), table)
    devs = [torch.from_numpy(h.reshape(-1)).cuda() for h in hosts]
    dst = torch.full((q * 16384,), float("nan"), dtype=torch.float32, device="cuda")
    bfz.pack_shard(plan, devs, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("off", [0, 1, 2, 3])
def test_pack_offset_bases(off):
    """Weights that start `off` floats past a 16-byte boundary: every row
    misalignment 0..3 meets widths that are and are not multiples of 4,
    right-edge tiles and single-row tiles."""
    dims = [(1, 129, 300), (2, 200, 257), (1, 77, 128), (1, 130, 131), (1, 1, 515)]
    _say("pack with weights offset by", off, "floats")
    rng = np.random.default_rng(100 + off)
    hosts = [rng.normal(0, 1, d).astype(np.float32) for d in dims]
    q, owned, table = oracle.plan(dims, 1, 0)
    want = oracle.pack(dims, hosts, table)
    plan = bfz.Plan(dims, 1, 0)
    devs = []
    for h in hosts:
        raw = torch.full((h.size + 8,), float("nan"), dtype=torch.float32, device="cuda")
        raw[off:off + h.size] = torch.from_numpy(h.reshape(-1)).cuda()
        devs.append(raw[off:off + h.size])
    assert all(d.data_ptr() % 16 == 4 * off for d in devs)
    dst = torch.full((q * 16384,), float("nan"), dtype=torch.float32, device="cuda")
    bfz.pack_shard(plan, devs, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_pack_segment_beyond_32bit_work_items():
    """One weight of 1024 x 1025 tiles (1,049,600 slots, 17.2G elements,
    69 GB a side): the fold runs four 1024-thread workgroups per slot, so
    this launch segment holds more work-items than one launch can count in
    32 bits and goes out in two launches.  Every tile must hold its block of
    the weight, bit for bit.  The fold is a pure layout copy, so the
    weight's own blocks are the reference; the values name their position
    (row-major index mod 2^24, exact in float32)."""
    H, W = 128 * 1024, 128 * 1025
    hb, wb = H // 128, W // 128
    plan = bfz.Plan([(1, H, W)], 1, 0)
    q = plan.shard_tiles
    assert q == hb * wb and q * 4 * 1024 >= 2 ** 32
    _say("pack of one", H, "x", W, "weight:", q, "slots in one segment")
    src = torch.empty(H * W, dtype=torch.float32, device="cuda")
    cols = torch.arange(W, dtype=torch.int64, device="cuda")
    for r0 in range(0, H, 1024):
        rows = torch.arange(r0, r0 + 1024, dtype=torch.int64, device="cuda")
        src.view(H, W)[r0:r0 + 1024] = ((rows[:, None] * W + cols[None, :]) % (1 << 24)).float()
    del cols, rows
    dst = torch.full((q * 16384,), float("nan"), dtype=torch.float32, device="cuda")
    bfz.pack_shard(plan, [src], dst)
    torch.cuda.synchronize()
    tiles = dst.view(hb, wb, 128, 128)
    blocks = src.view(hb, 128, wb, 128)
    for i0 in range(0, hb, 64):
        ok = torch.equal(tiles[i0:i0 + 64].view(torch.int32),
                         blocks[i0:i0 + 64].permute(0, 2, 1, 3).view(torch.int32))
        assert ok, ("tile rows", i0, i0 + 63)
    del tiles, blocks, src, dst
    torch.cuda.empty_cache()


@pytest.mark.parametrize("case", range(len(CASES)))
def test_unpack_matches_oracle(case):
    dims, D, rank = CASES[case]
    _say("unpack case", case, "D", D, "rank", rank, "weights", len(dims))
    rng = np.random.default_rng(100 + case)
    q, owned, table = oracle.plan(dims, D, rank)
    codes = rng.integers(0, 256, q * 16384).astype(np.uint8)
    scale = rng.uniform(0.1, 10, q).astype(np.float32)
    o8 = [np.full(d, 0x5A, dtype=np.uint8) for d in dims]
    osc = [np.full((d[0], -(-d[1] // 128), -(-d[2] // 128)), -7.0, dtype=np.float32) for d in dims]
    oracle.unpack(dims, codes, scale, table, o8, osc)
    plan = bfz.Plan(dims, D, rank)
    d8 = [torch.full((int(np.prod(d)),), 0x5A, dtype=torch.uint8, device="cuda") for d in dims]
    dsc = [torch.full((s.size,), -7.0, dtype=torch.float32, device="cuda") for s in osc]
    bfz.unpack_fp8(plan, torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(), d8, dsc)
    torch.cuda.synchronize()
    for p in range(len(dims)):
        assert np.array_equal(d8[p].cpu().numpy(), o8[p].reshape(-1)), p
        assert np.array_equal(dsc[p].cpu().numpy(), osc[p].reshape(-1)), p


def test_unpack_misaligned_destination():
    """A destination that starts 1 byte into its allocation takes the byte path."""
    dims = [(1, 256, 256)]
    _say("unpack into a misaligned destination")
    rng = np.random.default_rng(7)
    q, owned, table = oracle.plan(dims, 1, 0)
    codes = rng.integers(0, 256, q * 16384).astype(np.uint8)
    scale = np.ones(q, dtype=np.float32)
    o8 = [np.zeros(dims[0], dtype=np.uint8)]
    oracle.unpack(dims, codes, scale, table, o8, [np.zeros((1, 2, 2), np.float32)])
    plan = bfz.Plan(dims, 1, 0)
    raw = torch.zeros(256 * 256 + 1, dtype=torch.uint8, device="cuda")
    sc = torch.zeros(4, dtype=torch.float32, device="cuda")
    bfz.unpack_fp8(plan, torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(), [raw[1:]], [sc])
    torch.cuda.synchronize()
    assert np.array_equal(raw[1:].cpu().numpy(), o8[0].reshape(-1))


def _thresholds():
    """Smallest positive fp32 bit pattern the oracle maps to each code 1..126
    (the oracle's encoding is monotone in |y|), found by bisection."""
    thr = []
    for c in range(1, 127):
        lo, hi = 0, 0x7F800000
        while lo < hi:
            mid = (lo + hi) // 2
            y = np.array([mid], dtype=np.uint32).view(np.float32)
            if oracle.e4m3_encode(y)[0] >= c:
                hi = mid
            else:
                lo = mid + 1
        thr.append(lo)
    return thr


def test_e4m3_every_fp32_pattern():
    _say("E4M3 rounding over all 2^32 fp32 patterns")
    thr = torch.tensor(_thresholds(), dtype=torch.int64, device="cuda")
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    bad = 0
    for start in range(0, 1 << 32, chunk):
        bits = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda")
        x = bits.to(torch.int32).view(torch.float32)  # wraps to the signed pattern
        bfz.e4m3_encode(x, out)
        mag = bits & 0x7FFFFFFF
        want = torch.bucketize(mag, thr, right=True).to(torch.uint8)
        want = want | ((bits >> 31).to(torch.uint8) << 7)
        finite = mag < 0x7F800000
        bad += int(((out != want) & finite).sum())
        del bits, x, mag, want, finite
    assert bad == 0
