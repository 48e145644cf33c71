"""Pins of the oracle's E4M3 encoder and decoder (CPU only).

* hand-derived code values and roundings (tests/golden, each with its source);
* every finite fp32 bit pattern, clamped to +-448, against torch's own
  float8_e4m3fn cast (a library routine: round-to-nearest-even, OCP E4M3FN);
* structural facts: 127 ascending non-negative values, max 448, NaN slot.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                out.append(line.split())
    return out


def test_decode_golden(ora):
    rows = _rows("e4m3_codes.txt")
    assert len(rows) >= 20
    for code, s, e, m, val in rows:
        c = int(code, 16)
        assert (c >> 7, (c >> 3) & 15, c & 7) == (int(s), int(e), int(m))
        got = ora.e4m3_decode(c)
        assert got == float(val), (code, got, val)
        if float(val) == 0.0:
            assert np.signbit(got) == (int(s) == 1)


def test_encode_golden(ora):
    rows = _rows("e4m3_rounding.txt")
    ys = np.array([float(r[0]) for r in rows], dtype=np.float32)
    exp = np.array([int(r[1], 16) for r in rows], dtype=np.uint8)
    got = ora.e4m3_encode(ys)
    bad = [(float(y), hex(g), hex(x)) for y, g, x in zip(ys, got, exp) if g != x]
    assert not bad, bad


def test_value_table_structure(ora):
    vals = [ora.e4m3_decode(c) for c in range(127)]
    assert all(a < b for a, b in zip(vals, vals[1:]))
    assert vals[-1] == 448.0 and vals[0] == 0.0
    assert np.isnan(ora.e4m3_decode(0x7F)) and np.isnan(ora.e4m3_decode(0xFF))
    for c in range(127):
        assert ora.e4m3_decode(c | 0x80) == -vals[c]
    # every value re-encodes to its own code
    codes = np.arange(127, dtype=np.uint8)
    ys = np.array(vals, dtype=np.float32)
    assert np.array_equal(ora.e4m3_encode(ys), codes)
    assert np.array_equal(ora.e4m3_encode(-ys), codes | 0x80)


def _chunk_mismatches(ora, start, n, stride=1):
    bits = np.arange(start, start + n, stride, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    finite = np.isfinite(y)
    mine = ora.e4m3_encode(y)
    ref = torch.from_numpy(np.clip(y, -448.0, 448.0)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    bad = finite & (mine != ref)
    return int(bad.sum()), (bits[bad][:5].tolist() if bad.any() else [])


@pytest.mark.slow
def test_encode_exhaustive_vs_torch(ora):
    """Every one of the 2^32 fp32 bit patterns against torch's float8_e4m3fn
    cast after clamping to +-448; non-finite patterns skipped."""
    chunk = 1 << 26
    starts = [(s, 1) for s in range(0, 1 << 32, chunk)]
    n_thr = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with ThreadPoolExecutor(max_workers=os.cpu_count() or 4) as ex:
            res = list(ex.map(lambda a: _chunk_mismatches(ora, a[0], chunk, a[1]), starts))
    finally:
        torch.set_num_threads(n_thr)
    total = sum(r[0] for r in res)
    examples = [e for r in res for e in r[1]][:10]
    assert total == 0, (total, [hex(b) for b in examples])


def test_near_midpoint_flags(ora):
    # exactly on a midpoint, just off it, and far from it
    assert ora.e4m3_near_midpoint(1.0625)
    assert ora.e4m3_near_midpoint(np.float32(1.0625) * np.float32(1 + 5e-7))
    assert not ora.e4m3_near_midpoint(1.0625 * (1 + 5e-6))
    assert not ora.e4m3_near_midpoint(1.0)
    assert not ora.e4m3_near_midpoint(448.0)
    assert ora.e4m3_near_midpoint(-0.0146484375)
    # the window is relative to the midpoint: 5e-7 relative off 304 (between
    # 288 and 320) is near, 5e-7 absolute off 2^-10 (between 0 and 2^-9) is not
    assert ora.e4m3_near_midpoint(np.float32(304.0) * np.float32(1 + 5e-7))
    assert not ora.e4m3_near_midpoint(np.float32(2.0 ** -10 + 5e-7))
