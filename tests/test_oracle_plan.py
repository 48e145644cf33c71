"""Pins of the oracle's block-wise split (CPU only).

"A ZeRO Optimizer Design for Blockwise FP8 Quantization", section
"Block-wise split": the buffer is cut at 128x128 units, quantized dims are
padded to multiples of 128, and a lookup table keeps each unit's real
extent.  How units are dealt to ranks is not spelled out on the page (a
reading: contiguous equal quotas), so the rule itself is parity-unpinned;
what is pinned here, by brute force, is what any valid split must satisfy
and the counts the workload shapes fix.
"""
import itertools
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _enumerate_tiles(dims):
    """Every 128x128 unit of every param in fold order, with its extent."""
    out = []
    for p, (E, H, W) in enumerate(dims):
        hb, wb = -(-H // 128), -(-W // 128)
        for e, i, j in itertools.product(range(E), range(hb), range(wb)):
            out.append((p, e, i, j, min(128, H - 128 * i), min(128, W - 128 * j)))
    return out


def _random_dims(rng, n):
    return [(int(rng.integers(1, 4)), int(rng.integers(1, 700)), int(rng.integers(1, 700)))
            for _ in range(n)]


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_ownership(ora, seed):
    rng = np.random.default_rng(seed)
    dims = _random_dims(rng, int(rng.integers(1, 6)))
    allt = _enumerate_tiles(dims)
    T = len(allt)
    assert ora.total_tiles(dims) == T
    for D in range(1, 10):
        seen = []
        qs = set()
        for r in range(D):
            q, owned, table = ora.plan(dims, D, r)
            qs.add(q)
            assert q * D >= T and (q - 1) * D < T  # the smallest equal quota
            assert 0 <= owned <= q
            rows = [tuple(int(x) for x in row) for row in table]
            assert all(row[0] >= 0 for row in rows[:owned])
            assert all(row == (-1, 0, 0, 0, 0, 0) for row in rows[owned:])
            seen.extend(rows[:owned])
        assert len(qs) == 1
        # every unit owned exactly once, and ranks hold consecutive ranges
        assert seen == allt


def test_toy_walkthrough(ora):
    lines = [ln.split("#")[0].split() for ln in open(os.path.join(GOLDEN, "zero1_toy_layout.txt"))]
    lines = [ln for ln in lines if ln]
    dims = [tuple(int(x) for x in lines[0][1:])]
    D = int(lines[1][1])
    for r, first, owned_want in (tuple(int(x) for x in ln) for ln in lines[2:]):
        q, owned, table = ora.plan(dims, D, r)
        assert owned == owned_want and q == 4
        glob = [i * 4 + j for (_, _, i, j, _, _) in table]
        assert glob == list(range(first, first + owned))


def test_workload_counts(ora):
    # Dense LLM: 32 layers x {4 of 4096x4096, 2 of 4096x11008, 1 of 11008x4096}
    dense = [(1, 4096, 4096)] * 4 + [(1, 4096, 11008)] * 2 + [(1, 11008, 4096)]
    dims = dense * 32
    per_layer = 4 * 32 * 32 + 2 * 32 * 86 + 86 * 32  # 11008/128 = 86
    assert ora.total_tiles(dims) == 32 * per_layer == 395264
    q, owned, table = ora.plan(dims, 8, 0)
    assert q == owned == 49408
    assert set(table[:, 0]) == set(range(28))  # rank 0 holds layers 0-3 whole
    # MoE experts: 256 x gate/up (7168x2048) and down (2048x7168), D = 32
    moe = [(256, 7168, 2048), (256, 7168, 2048), (256, 2048, 7168)]
    assert ora.total_tiles(moe) == 3 * 256 * 56 * 16 == 688128
    q, owned, table = ora.plan(moe, 32, 0)
    assert q == owned == 21504
    assert (table[:, 0] == 0).all() and table[-1, 1] == 23  # gate of experts 0-23


def test_invalid_arguments(ora):
    with pytest.raises(ValueError):
        ora.plan([(1, 10, 10)], 0, 0)
    with pytest.raises(ValueError):
        ora.plan([(1, 10, 10)], 4, 4)
    with pytest.raises(ValueError):
        ora.plan([(1, 0, 10)], 1, 0)
    with pytest.raises(ValueError):
        ora.plan([(1, 10, 10)], 2, -1)


def test_more_ranks_than_tiles(ora):
    dims = [(1, 200, 130)]  # 2 x 2 = 4 tiles
    owned_all = []
    for r in range(7):
        q, owned, table = ora.plan(dims, 7, r)
        assert q == 1
        owned_all.append(owned)
    assert owned_all == [1, 1, 1, 1, 0, 0, 0]


# ---- the param-wise split ----------------------------------------------------

def _opt_makespan(sizes, D):
    best = None
    for assign in itertools.product(range(D), repeat=len(sizes)):
        loads = [0] * D
        for s, b in zip(sizes, assign):
            loads[b] += s
        m = max(loads)
        best = m if best is None else min(best, m)
    return best


def test_paramwise_graham_worst_case(ora):
    """Graham's tight example for largest-first greedy on 2 buckets (R. L.
    Graham, "Bounds on multiprocessing timing anomalies", SIAM J. Appl. Math.
    17, 1969): sizes 3, 3, 2, 2, 2 -- greedy reaches 7 where 6 is optimal,
    exactly the bound 4/3 - 1/(3D) times the optimum."""
    bop, be = ora.paramwise_split([(1, 1, s) for s in (3, 3, 2, 2, 2)], 2)
    assert list(bop) == [0, 1, 0, 1, 0] and sorted(be) == [5, 7]


@pytest.mark.parametrize("seed", range(30))
def test_paramwise_brute_force(ora, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 8))
    D = int(rng.integers(1, 4))
    dims = [(int(rng.integers(1, 3)), int(rng.integers(1, 20)), int(rng.integers(1, 20)))
            for _ in range(n)]
    sizes = [E * H * W for E, H, W in dims]
    bop, be = ora.paramwise_split(dims, D)
    assert ((bop >= 0) & (bop < D)).all()
    for b in range(D):
        assert be[b] == sum(s for s, x in zip(sizes, bop) if x == b)
    opt = _opt_makespan(sizes, D)
    assert opt <= be.max() <= (4 / 3 - 1 / (3 * D)) * opt + 1e-9
    # largest first: a weight never lands on a bucket that was already the
    # fullest when it was placed, so no bucket exceeds the rest by more than
    # its own smallest weight
    for b in range(D):
        mine = [s for s, x in zip(sizes, bop) if x == b]
        if mine:
            assert be[b] - min(mine) <= min(be) or D == 1


def test_paramwise_too_few_weights(ora):
    """The page's second drawback: with fewer weights than ranks some
    buckets stay empty, and every rank is padded to a whole weight."""
    moe = [(256, 7168, 2048), (256, 7168, 2048), (256, 2048, 7168)]
    bop, be = ora.paramwise_split(moe, 32)
    assert sorted(bop) == [0, 1, 2] and (be == 0).sum() == 29
    assert be.max() == 256 * 7168 * 2048
