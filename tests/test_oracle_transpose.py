"""Pins of the oracle's transposed power-of-two requantization (CPU only).

"FP8-Flow-MoE", section 3.1: with scales restricted to powers of two,
re-quantizing a tensor in another layout (its transpose, grouped along the
other dimension) only moves exponent bits, so it adds no error -- unlike the
dequantize -> transpose -> quantize route with arbitrary scales, where the
second rounding lands on a different grid.  Pins:

* lossless: every element of the transposed copy decodes to exactly the
  value the tile decoded to;
* torch's own route (float8_e4m3fn decode, .T, per-group power-of-two
  scale, float8_e4m3fn encode) gives the same codes and scales;
* group scales are the tight power of two of the group's amax and never
  exceed the tile's;
* with amax/448 scales the same route is lossy -- the double quantization
  error the power-of-two restriction removes.
"""
import numpy as np
import pytest
import torch

T = 16384


def _decode_all(ora):
    return np.array([ora.e4m3_decode(c) for c in range(256)], dtype=np.float64)


def _quantized_weight(ora, dims, seed, pow2=True, zero_cols=False):
    """Row-major weights -> (table, tile-major codes, scales) via the oracle."""
    rng = np.random.default_rng(seed)
    ws = []
    for E, H, W in dims:
        x = rng.normal(0, 1, (E, H, W)) * 10.0 ** rng.uniform(-3, 1, (E, H, 1))
        if zero_cols:
            x[:, :, ::5] = 0.0
        ws.append(x.astype(np.float32))
    q, owned, table = ora.plan(dims, 1, 0)
    shard = ora.pack(dims, ws, table)
    codes, scale, _ = ora.quant_tiles(shard, pow2=pow2)
    return table, codes, scale


def _pow2_tight(amax):
    """Smallest 2^T with 448 * 2^T >= amax, T >= -149 (exact comparisons)."""
    T = int(np.floor(np.log2(amax / 448.0))) - 1
    T = max(T, -149)
    while 448.0 * 2.0 ** T < amax:
        T += 1
    return 2.0 ** T


def _run(ora, dims, table, codes, scale):
    dt = [np.full((E, W, H), 0xAA, dtype=np.uint8) for E, H, W in dims]
    ds = [np.full((E, W, -(-H // 128)), -1.0, dtype=np.float32) for E, H, W in dims]
    ora.transpose_pow2(dims, codes, scale, table, dt, ds)
    return dt, ds


SHAPES = [[(1, 256, 384)], [(2, 300, 129), (1, 77, 513)], [(1, 128, 1000), (3, 129, 130)]]


@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_transpose_is_lossless(ora, case):
    dims = SHAPES[case]
    dec = _decode_all(ora)
    table, codes, scale = _quantized_weight(ora, dims, 10 + case, zero_cols=case == 1)
    dt, ds = _run(ora, dims, table, codes, scale)
    for s, (p, e, i, j, vr, vc) in enumerate(table):
        E, H, W = dims[p]
        tile = codes[s * T:(s + 1) * T].reshape(128, 128)[:vr, :vc]
        vals = dec[tile] * float(scale[s])                            # [r, c]
        out = dt[p][e, 128 * j:128 * j + vc, 128 * i:128 * i + vr]     # [c, r]
        g = ds[p][e, 128 * j:128 * j + vc, i].astype(np.float64)        # per c
        back = dec[out] * g[:, None]
        assert np.array_equal(back, vals.T), (case, s)
        # tight, power of two, never above the tile's scale
        amax = np.abs(vals).max(axis=0)
        for c in range(vc):
            if amax[c] == 0:
                assert g[c] == 1.0 and (out[c] == 0).all()
            else:
                assert g[c] == _pow2_tight(amax[c]) and g[c] <= scale[s]


@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_transpose_matches_torch_route(ora, case):
    dims = SHAPES[case]
    table, codes, scale = _quantized_weight(ora, dims, 20 + case)
    dt, ds = _run(ora, dims, table, codes, scale)
    for s, (p, e, i, j, vr, vc) in enumerate(table):
        tile = torch.from_numpy(codes[s * T:(s + 1) * T].reshape(128, 128)[:vr, :vc].copy())
        vals = tile.view(torch.float8_e4m3fn).to(torch.float64) * float(scale[s])
        vt = vals.T.contiguous()                                       # [c, r]
        amax = vt.abs().amax(dim=1)
        g = torch.tensor([_pow2_tight(a) if a > 0 else 1.0 for a in amax.tolist()],
                         dtype=torch.float64)
        y = (vt / g[:, None]).to(torch.float32).clamp(-448, 448)
        want = y.to(torch.float8_e4m3fn).view(torch.uint8)
        want[amax == 0] = 0
        got = torch.from_numpy(dt[p][e, 128 * j:128 * j + vc, 128 * i:128 * i + vr].copy())
        assert torch.equal(got, want), (case, s)
        assert np.array_equal(ds[p][e, 128 * j:128 * j + vc, i], g.numpy().astype(np.float32))


def test_arbitrary_scales_are_not_lossless(ora):
    """The same dequantize -> transpose -> quantize route with amax/448
    scales does move values: the double quantization error the section
    describes."""
    dims = [(1, 256, 256)]
    dec = _decode_all(ora)
    table, codes, scale = _quantized_weight(ora, dims, 30, pow2=False)
    moved = 0
    for s in range(len(table)):
        vals = dec[codes[s * T:(s + 1) * T].reshape(128, 128)] * float(scale[s])
        vt = vals.T
        g = np.abs(vt).max(axis=1).astype(np.float32) / np.float32(448.0)
        y = (vt / g[:, None]).astype(np.float32)
        back = dec[ora.e4m3_encode(y)] * g[:, None]
        moved += int((back != vt).sum())
    assert moved > 1000
