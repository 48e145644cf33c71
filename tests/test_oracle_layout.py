"""Pins of the oracle's fold (pack) and unfold (unpack), CPU only.

"A ZeRO Optimizer Design for Blockwise FP8 Quantization", section
"Parameter layout transform": fold makes every 128x128 unit of a row-major
weight contiguous, units in (expert, tile row, tile column) order; unfold is
its inverse, for the FP8 weights and for the scale grid.  The pins use
torch's im2col / col2im (F.unfold / F.fold with a 128x128 kernel and
stride), an independent library route to the same tiling; ragged weights
are zero-padded to multiples of 128 first (section "Block-wise split").
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

SHAPES = [(1, 256, 384), (2, 128, 128), (1, 129, 300), (3, 200, 257), (1, 1, 1), (2, 383, 128)]


def _torch_tiles(x):
    """x: (E, H, W) float tensor -> (E * hb * wb, 128, 128) via im2col."""
    E, H, W = x.shape
    hp, wp = -(-H // 128) * 128, -(-W // 128) * 128
    xp = F.pad(x, (0, wp - W, 0, hp - H))
    cols = F.unfold(xp.unsqueeze(1), kernel_size=128, stride=128)  # (E, 16384, L)
    return cols.transpose(1, 2).reshape(-1, 128, 128)


@pytest.mark.parametrize("shape", SHAPES)
def test_pack_matches_im2col(ora, shape):
    rng = np.random.default_rng(sum(shape))
    x = rng.normal(0, 1, shape).astype(np.float32)
    q, owned, table = ora.plan([shape], 1, 0)
    got = ora.pack([shape], [x], table).reshape(-1, 128, 128)
    ref = _torch_tiles(torch.from_numpy(x)).numpy()
    assert got.shape == ref.shape
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))  # pads are +0.0


@pytest.mark.parametrize("shape", SHAPES)
def test_unpack_matches_col2im(ora, shape):
    E, H, W = shape
    rng = np.random.default_rng(100 + sum(shape))
    q, owned, table = ora.plan([shape], 1, 0)
    codes = rng.integers(0, 256, q * 16384).astype(np.uint8)
    scale = rng.uniform(0.5, 2, q).astype(np.float32)
    dst = np.full(shape, 0xAA, dtype=np.uint8)
    hb, wb = -(-H // 128), -(-W // 128)
    dsc = np.zeros((E, hb, wb), dtype=np.float32)
    ora.unpack([shape], codes, scale, table, [dst], [dsc])
    cols = torch.from_numpy(codes.astype(np.float32)).view(E, hb * wb, 16384).transpose(1, 2)
    full = F.fold(cols, output_size=(hb * 128, wb * 128), kernel_size=128, stride=128)
    ref = full[:, 0, :H, :W].numpy().astype(np.uint8)
    assert np.array_equal(dst, ref)
    assert np.array_equal(dsc, scale.reshape(E, hb, wb))


def test_round_trip_multi_param_multi_rank(ora):
    dims = [(2, 300, 200), (1, 128, 640), (3, 129, 129)]
    rng = np.random.default_rng(5)
    xs = [rng.integers(0, 256, d).astype(np.uint8) for d in dims]
    srcs = [x.astype(np.float32) for x in xs]
    D = 3
    outs = [np.zeros(d, dtype=np.uint8) for d in dims]
    scs = [np.full((d[0], -(-d[1] // 128), -(-d[2] // 128)), -1.0, dtype=np.float32) for d in dims]
    for r in range(D):
        q, owned, table = ora.plan(dims, D, r)
        shard = ora.pack(dims, srcs, table)
        assert (shard[owned * 16384:] == 0).all()
        codes = shard.astype(np.uint8)
        ora.unpack(dims, codes, np.arange(q, dtype=np.float32) + 100 * r, table, outs, scs)
    for x, o in zip(xs, outs):
        assert np.array_equal(x, o)
    # every scale cell written once, by the rank that owns that unit
    got = np.concatenate([s.reshape(-1) for s in scs])
    want = np.concatenate([np.arange(ora.plan(dims, D, r)[1], dtype=np.float32) + 100 * r
                           for r in range(D)])
    assert np.array_equal(got, want)
