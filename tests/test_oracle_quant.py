"""Pins of the oracle's per-tile E4M3 quantization (CPU only).

From "FP8-Flow-MoE" section 3.1: one scale per tile, s = amax/448, codes
are x/s rounded to the nearest E4M3 value, dequantization multiplies by s,
and re-quantizing a dequantized tile in the same layout changes nothing.
Pins: the largest code of every nonzero tile decodes to 448; the
dequantization error is within half an E4M3 spacing; idempotence; tiles
built from exact grid multiples give known codes; the all-zero guard
(lpnh.cn essay, sections 4.2 / 5.1); and agreement, away from rounding
midpoints, with the multiply-by-448/amax form of the 128x128 block
quantizer sketched in "FP8 training: core scaling strategies", section 3.2,
rounded by torch's float8_e4m3fn cast.
"""
import numpy as np
import pytest
import torch

T = 16384


def _decode_all(ora):
    return np.array([ora.e4m3_decode(c) for c in range(256)], dtype=np.float64)


def _tiles(seed, n_tiles, kind):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.normal(0, 0.02, n_tiles * T)
    elif kind == "heavy":
        x = rng.standard_t(3, n_tiles * T) * 1e-3
    elif kind == "wide":  # many binades inside one tile
        x = rng.normal(0, 1, n_tiles * T) * 10.0 ** rng.uniform(-12, 3, n_tiles * T)
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


@pytest.mark.parametrize("kind", ["normal", "heavy", "wide"])
def test_invariants(ora, kind):
    dec = _decode_all(ora)
    p = _tiles(1, 6, kind)
    p[5 * T:] = 0.0  # one all-zero tile
    p[4 * T + 777] = -3.5  # amax at a negative value
    codes, scale, near = ora.quant_tiles(p)
    for t in range(6):
        x = p[t * T:(t + 1) * T].astype(np.float64)
        c = codes[t * T:(t + 1) * T]
        if t == 5:
            assert scale[t] == 1.0 and (c == 0).all() and (near[t * T:] == 0).all()
            continue
        amax = np.abs(x).max()
        assert scale[t] == np.float32(np.float32(amax) / np.float32(448.0))
        assert np.abs(dec[c]).max() == 448.0
        k = int(np.argmax(np.abs(x)))
        assert c[k] == (0xFE if x[k] < 0 else 0x7E)
        # error bound: half the E4M3 spacing at |y|, times the scale, plus
        # the two binary32 roundings (scale and quotient)
        s = float(scale[t])
        y = np.abs(x) / s
        e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
        spacing = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))
        err = np.abs(x - dec[c] * s)
        bound = 0.5 * spacing * s * (1 + 2.0 ** -20) + np.abs(x) * 2.0 ** -22
        assert (err <= bound).all(), float((err - bound).max())
        # sign of every code is the sign of the value
        assert ((c >= 0x80) == np.signbit(x)).all()


@pytest.mark.parametrize("kind", ["normal", "heavy", "wide"])
def test_same_layout_requant_is_idempotent(ora, kind):
    dec = _decode_all(ora)
    p = _tiles(2, 4, kind)
    codes, scale, _ = ora.quant_tiles(p)
    deq = (dec[codes] * np.repeat(scale.astype(np.float64), T)).astype(np.float32)
    codes2, scale2, _ = ora.quant_tiles(deq)
    assert np.array_equal(codes2, codes)
    assert np.all(np.abs(scale2.astype(np.float64) / scale - 1) <= 2.0 ** -23)


def test_exact_grid_tile(ora):
    """Every finite code times a power-of-two scale, plus exact midpoints."""
    dec = _decode_all(ora)
    s = 2.0 ** -10
    vals, want = [], []
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        vals.append(dec[c] * s)
        want.append(c)
    for c in range(126):  # midpoints between neighbours: tie to even code
        for sign in (0, 0x80):
            mid = 0.5 * (dec[c] + dec[c + 1]) * s
            vals.append(-mid if sign else mid)
            want.append((c if c % 2 == 0 else c + 1) | sign)
    x = np.zeros(T, dtype=np.float32)
    x[:len(vals)] = vals
    codes, scale, near = ora.quant_tiles(x)
    assert scale[0] == np.float32(s)  # amax is 448 s, so the scale is s exactly
    assert np.array_equal(codes[:len(want)], np.array(want, dtype=np.uint8))
    assert (codes[len(want):] == 0).all()
    assert near[254:len(want)].all()


def test_block_quantize_multiply_form(ora):
    """The 128x128 block quantizer of the FP8 scaling-strategies page scales
    by 448/amax and rounds; with torch's E4M3 cast as the rounding it agrees
    with the oracle except where the quotient sits next to a midpoint."""
    p = _tiles(3, 8, "normal")
    codes, scale, near = ora.quant_tiles(p)
    x = torch.from_numpy(p).view(8, 128, 128)
    amax = x.abs().amax(dim=(1, 2), keepdim=True)
    y = (x * (448.0 / amax)).clamp(-448.0, 448.0)
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(-1).numpy()
    diff = ref != codes
    assert diff.sum() <= 50
    assert near[diff].all()


def test_zero_tile_guard_and_padding(ora):
    x = np.zeros(2 * T, dtype=np.float32)
    x[T + 5] = 1e-30  # a tiny but nonzero tile
    codes, scale, _ = ora.quant_tiles(x)
    assert scale[0] == 1.0 and (codes[:T] == 0).all()
    assert scale[1] == np.float32(np.float32(1e-30) / np.float32(448.0))
    assert codes[T + 5] == 0x7E and (np.delete(codes[T:], 5) == 0).all()


def test_scale_underflow_floor(ora):
    """A nonzero tile whose amax / 448 rounds to zero in binary32 (amax at
    most 224 * 2^-149) takes the scale 2^-149 instead of dividing by zero:
    x / 2^-149 is then an exact integer of magnitude <= 224, so the codes
    are torch's E4M3 cast of those integers (signed zero kept).  One step
    above the threshold the plain amax / 448 applies again (and rounds to
    the same 2^-149)."""
    tiny = 2.0 ** -149
    rng = np.random.default_rng(9)
    x = np.zeros(3 * T, dtype=np.float32)
    x[:T] = (rng.integers(-100, 101, T) * tiny).astype(np.float32)
    x[0], x[1] = np.float32(100 * tiny), np.float32(-0.0)
    x[T + 17] = np.float32(-224 * tiny)                 # the tie: 224 / 448 rounds to 0
    x[2 * T + 5] = np.float32(225 * tiny)               # just above it
    x[2 * T + 6] = np.float32(-3 * tiny)
    codes, scale, _ = ora.quant_tiles(x)
    assert np.float32(np.float32(224 * tiny) / np.float32(448.0)) == 0.0
    assert scale[0] == np.float32(tiny) and scale[1] == np.float32(tiny)
    assert scale[2] == np.float32(np.float32(225 * tiny) / np.float32(448.0)) == np.float32(tiny)
    y = torch.from_numpy((x.astype(np.float64) / tiny).astype(np.float32))
    want = y.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, want)
    assert codes[1] == 0x80 and codes[T + 17] == 0xF6  # -224 = -1.75 * 2^7: E = 14, M = 6


# ---- power-of-two scales ------------------------------------------------------

@pytest.mark.parametrize("kind", ["normal", "heavy", "wide"])
def test_pow2_invariants(ora, kind):
    """Power-of-two tile scales ("FP8-Flow-MoE" §3.1): the scale is 2^T,
    the smallest power of two with 448 * 2^T >= amax, so the largest code
    decodes into [224, 448]; every quotient x / 2^T is exact, so the codes
    equal torch's E4M3 cast of the exactly scaled values."""
    dec = _decode_all(ora)
    p = _tiles(4, 6, kind)
    p[5 * T:] = 0.0
    codes, scale, _ = ora.quant_tiles(p, pow2=True)
    for t in range(6):
        x = p[t * T:(t + 1) * T].astype(np.float64)
        c = codes[t * T:(t + 1) * T]
        s = float(scale[t])
        if t == 5:
            assert s == 1.0 and (c == 0).all()
            continue
        m, e = np.frexp(s)
        assert m == 0.5  # a power of two
        amax = np.abs(x).max()
        assert 448 * s >= amax and (448 * s / 2 < amax or s == 2.0 ** -149)
        top = np.abs(dec[c]).max()
        assert 224 <= top <= 448
        y = torch.from_numpy((x / s).astype(np.float32))  # exact: s is a power of two
        ref = y.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ref, c)


@pytest.mark.parametrize("kind", ["normal", "wide"])
def test_pow2_requant_is_exactly_idempotent(ora, kind):
    dec = _decode_all(ora)
    p = _tiles(5, 4, kind)
    codes, scale, _ = ora.quant_tiles(p, pow2=True)
    deq = (dec[codes] * np.repeat(scale.astype(np.float64), T)).astype(np.float32)
    assert np.array_equal(deq.astype(np.float64), dec[codes] * np.repeat(scale.astype(np.float64), T))
    codes2, scale2, _ = ora.quant_tiles(deq, pow2=True)
    assert np.array_equal(scale2, scale) and np.array_equal(codes2, codes)


def test_pow2_scale_edges(ora):
    assert ora.pow2_scale(448.0) == 1.0
    assert ora.pow2_scale(448.0001) == 2.0
    assert ora.pow2_scale(224.0) == 0.5
    assert ora.pow2_scale(224.0001) == 1.0
    assert ora.pow2_scale(448.0 * 2.0 ** -20) == 2.0 ** -20
    assert ora.pow2_scale(2.0 ** -149) == 2.0 ** -149  # the clamp
    assert ora.pow2_scale(3.0e38) == 2.0 ** 120
