"""The seeded input generator (synth/), CPU side.

The generator holds none of the method's arithmetic; these checks pin its
own math and its counter-based contract, so a wrong series term or a
broken slice shows up here rather than as a puzzling parity failure:
- ln, exp, sqrt and cos(2 pi u) written from their series / Newton
  definitions agree with the C library to a few ulps (exp: about k ulps
  after its binary64 reduction x = k ln2 + r);
- normal and Student-t(3) draws have the moments / probabilities of their
  distributions (5-sigma statistical bounds);
- any slice of a stream regenerates alone (value k depends only on k)."""
import math

import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def L():
    return synth.lib()


def _ulps(a, b):
    return abs(a - b) / math.ulp(b) if b != 0 else abs(a) / math.ulp(1.0)


def test_ln_matches_libm(L):
    xs = np.concatenate([np.geomspace(1e-300, 1e300, 4001), np.linspace(0.5, 2.0, 2001),
                         [1.0, 2.0, 0.5, math.e, 1 + 2 ** -40]])
    worst = max(_ulps(L.synth_ln(float(x)), math.log(x)) if abs(math.log(x)) > 1e-3
                else abs(L.synth_ln(float(x)) - math.log(x)) / 1e-19 for x in xs)
    assert worst <= 4, worst


def test_exp_matches_libm(L):
    # the reduction x = k ln2 + r uses ln2 in binary64 only, so the relative
    # error grows with k (about k ulps); the generator calls exp on
    # ln(10) * [-5, -2] (per-expert factors 10^U(-5, -2)), k <= 17
    xs = np.linspace(-30, 30, 6001)
    worst = max(_ulps(L.synth_exp(float(x)), math.exp(x)) for x in xs)
    assert worst <= 24, worst
    xs = np.linspace(-700, 700, 4001)
    worst_rel = max(abs(L.synth_exp(float(x)) / math.exp(x) - 1) for x in xs)
    assert worst_rel <= 2e-13, worst_rel


def test_sqrt_matches_libm(L):
    xs = np.concatenate([np.geomspace(1e-300, 1e300, 4001), np.linspace(0.01, 100, 2001)])
    worst = max(_ulps(L.synth_sqrt(float(x)), math.sqrt(x)) for x in xs)
    assert worst <= 2, worst


def test_cos_turns_matches_libm(L):
    us = np.concatenate([np.linspace(0.0, 1.0, 8001, endpoint=False), [0.125, 0.25, 0.375, 0.5]])
    # both sides round 2 pi u (libm's argument too), so compare absolutely
    worst = max(abs(L.synth_cos_turns(float(u)) - math.cos(2 * math.pi * u)) for u in us)
    assert worst <= 1e-15, worst


def test_uniform_is_open_interval_and_flat(L):
    k = synth.key(7, 1, 2, 3)
    u = np.array([L.synth_uniform(k, j) for j in range(200000)])
    assert u.min() > 0.0 and u.max() < 1.0
    n = len(u)
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / n)
    hist = np.histogram(u, bins=20, range=(0, 1))[0]
    assert np.all(np.abs(hist - n / 20) < 5 * math.sqrt(n / 20))


def test_normal_moments():
    n = 400000
    r = synth.recipe(synth.NORMAL, synth.key(1, 2, 3, 4), 1, n, scale=1.0)
    z = synth.fill_host(r, 0, n).astype(np.float64)
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2 / n)
    assert abs(np.mean(np.abs(z) < 1.0) - 0.682689492) < 5 * math.sqrt(0.25 / n)


def test_student_t3_probabilities():
    # Student-t with 3 degrees of freedom: P(|T| < 1) = 2 F(1) - 1 with
    # F(t) = 1/2 + (1/pi) (t / (sqrt 3 (1 + t^2/3)) + atan(t / sqrt 3))
    n = 200000
    r = synth.recipe(synth.T3, synth.key(5, 6, 7, 8), 1, n, scale=1.0)
    t = synth.fill_host(r, 0, n).astype(np.float64)

    def cdf(x):
        s3 = math.sqrt(3.0)
        return 0.5 + (x / (s3 * (1 + x * x / 3)) + math.atan(x / s3)) / math.pi

    for a in (0.5, 1.0, 2.0, 4.0):
        p = 2 * cdf(a) - 1
        got = np.mean(np.abs(t) < a)
        assert abs(got - p) < 5 * math.sqrt(p * (1 - p) / n), (a, got, p)
    assert abs(np.median(t)) < 0.01


def test_t3_squared_is_square_of_t3():
    n = 5000
    k = synth.key(9, 9, 9, 9)
    t = synth.fill_host(synth.recipe(synth.T3, k, 1, n, scale=1e-3), 0, n).astype(np.float64)
    t2 = synth.fill_host(synth.recipe(synth.T3_SQUARED, k, 1, n, scale=1e-3), 0, n)
    # both round the same binary64 draw; the square is taken before rounding
    assert np.allclose(t2, t * t, rtol=2 ** -22, atol=0)
    assert (t2 >= 0).all()


def test_slices_regenerate_alone():
    r = synth.recipe(synth.T3, synth.key(3, 1, 4, 1), 33, 77, scale=0.5, zero_tile_prob=0.3,
                     zero_key=synth.key(3, 1, 4, 2))
    whole = synth.fill_host(r, 0, 33 * 77 * 2)
    for lo, hi in ((0, 1), (5, 400), (1000, 5082), (33 * 77, 33 * 77 * 2)):
        assert np.array_equal(synth.fill_host(r, lo, hi).view(np.uint32),
                              whole[lo:hi].view(np.uint32))
    # rectangles of expert 1 are the same values, row by row
    rect = synth.fill_rect_host(r, 1, 3, 20, 10, 50)
    base = 33 * 77
    want = np.stack([whole[base + (3 + a) * 77 + 10: base + (3 + a) * 77 + 60] for a in range(20)])
    assert np.array_equal(rect.view(np.uint32), want.view(np.uint32))


def test_zero_tiles_are_whole_tiles():
    H, W = 300, 260
    r = synth.recipe(synth.NORMAL, synth.key(2, 2, 2, 2), H, W, scale=1.0, zero_tile_prob=0.4,
                     zero_key=synth.key(2, 2, 2, 3))
    a = synth.fill_host(r, 0, H * W).reshape(H, W)
    zero_tiles = 0
    for i in range(0, H, 128):
        for j in range(0, W, 128):
            blk = a[i:i + 128, j:j + 128]
            if (blk == 0).all():
                zero_tiles += 1
            else:
                assert (blk != 0).mean() > 0.99
    assert 0 < zero_tiles < 9
