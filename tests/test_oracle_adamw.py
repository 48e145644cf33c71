"""Pins of the oracle's AdamW (CPU only).

The AdamW step of the Int8AdamW optimizer in the lpnh.cn optimizer-state
quantization essay (section 4.3) is checked against

* closed forms: the first step from zero moments, and a warm state chosen so
  that the bias-corrected moments equal g and g^2 at any step t;
* torch.optim.AdamW (a library routine) with weight_decay = 0, where the
  two updates coincide mathematically;
* with weight_decay != 0, the exact size of the one intended difference:
  the page decays the already-updated parameter, torch the old one;
* invariants: zero padding stays +0.0, v >= 0.
"""
import numpy as np
import pytest
import torch

HP_SETS = [
    dict(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1),
    dict(lr=5e-2, beta1=0.8, beta2=0.99, eps=1e-3, weight_decay=0.5),
    dict(lr=1e-3, beta1=0.5, beta2=0.999, eps=1e-6, weight_decay=0.0),
]


def _ulp(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(x).astype(np.float64)


def _close(got, ref, ulps, abs_tol=0.0, scale=None):
    """|got - ref| <= ulps * ulp(scale) + abs_tol, scale defaulting to ref."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    lim = ulps * _ulp(ref if scale is None else scale) + abs_tol
    bad = err > lim
    assert not bad.any(), (int(bad.sum()), got[bad][:4], ref[bad][:4])


def _inputs(n, g_sigma, seed):
    rng = np.random.default_rng(seed)
    p = rng.normal(0, 0.02, n).astype(np.float32)
    g = rng.normal(0, g_sigma, n).astype(np.float32)
    return p, g


@pytest.mark.parametrize("hpk", range(len(HP_SETS)))
@pytest.mark.parametrize("g_sigma", [1e-3, 1e-8, 3.0])
def test_first_step_closed_form(ora, hpk, g_sigma):
    h = HP_SETS[hpk]
    p0, g = _inputs(20000, g_sigma, 10 + hpk)
    p = p0.copy()
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    ora.adamw(p, g, m, v, ora.hparams(step=1, **h))
    gd = g.astype(np.float64)
    b1, b2, lr, eps, wd = h["beta1"], h["beta2"], h["lr"], h["eps"], h["weight_decay"]
    _close(m, (1 - b1) * gd, 2)
    _close(v, (1 - b2) * gd * gd, 3)
    p_ref = (p0.astype(np.float64) - lr * gd / (np.abs(gd) + eps)) * (1 - lr * wd)
    # the update term lr*g/(|g|+eps) carries ~10 roundings of relative 2^-24
    _close(p, p_ref, 3, abs_tol=lr * 2e-6)


@pytest.mark.parametrize("t", [2, 11, 1000])
@pytest.mark.parametrize("hpk", range(len(HP_SETS)))
def test_warm_state_closed_form(ora, t, hpk):
    h = HP_SETS[hpk]
    b1, b2, lr, eps, wd = h["beta1"], h["beta2"], h["lr"], h["eps"], h["weight_decay"]
    p0, g = _inputs(20000, 1e-3, 100 + t)
    gd = g.astype(np.float64)
    # moments of a constant gradient after t-1 steps: (1-b^(t-1)) g, (1-b^(t-1)) g^2
    m = ((1 - b1 ** (t - 1)) * gd).astype(np.float32)
    v = ((1 - b2 ** (t - 1)) * gd * gd).astype(np.float32)
    p = p0.copy()
    ora.adamw(p, g, m, v, ora.hparams(step=t, **h))
    _close(m, (1 - b1 ** t) * gd, 4)
    _close(v, (1 - b2 ** t) * gd * gd, 6)
    p_ref = (p0.astype(np.float64) - lr * gd / (np.abs(gd) + eps)) * (1 - lr * wd)
    # bias correction divides rounding noise by (1-b^t): at t=2, b1=0.9 that is 1/0.19
    rel = 40 * 2.0 ** -24 / min(1 - b1 ** t, 1 - b2 ** t) ** 0.5
    _close(p, p_ref, 3, abs_tol=lr * rel)


def _torch_adamw(p0, grads, h):
    p = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([p], lr=h["lr"], betas=(h["beta1"], h["beta2"]), eps=h["eps"],
                            weight_decay=h["weight_decay"], foreach=False, fused=False)
    for g in grads:
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    st = opt.state[p]
    return (p.detach().numpy().copy(), st["exp_avg"].numpy().copy(),
            st["exp_avg_sq"].numpy().copy())


def test_matches_torch_adamw_without_decay(ora):
    h = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)
    rng = np.random.default_rng(7)
    n = 50000
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    grads = [rng.normal(0, 1e-3, n).astype(np.float32) for _ in range(3)]
    tp, tm, tv = _torch_adamw(p0, grads, h)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    m_scale = np.zeros(n)
    v_scale = np.zeros(n)
    for t, g in enumerate(grads, start=1):
        # torch forms m by lerp, m + (1-b1)(g - m), whose rounding is relative
        # to the operands rather than to the result, and may fuse
        # multiply-adds: bound each step's error by its operands' size
        m_scale = np.maximum(m_scale, np.abs(m) + np.abs(g))
        v_scale = np.maximum(v_scale, np.abs(v) + g.astype(np.float64) ** 2)
        ora.adamw(p, g, m, v, ora.hparams(step=t, **h))
    _close(m, tm, 4, scale=m_scale)
    _close(v, tv, 4, scale=v_scale)
    _close(p, tp, 2, abs_tol=h["lr"] * 1e-5)


def test_weight_decay_placement_vs_torch(ora):
    """The page decays the updated parameter: p' = (p - u)(1 - lr wd);
    torch decays the old one: p' = p (1 - lr wd) - u.  The difference is
    exactly lr*wd*u, with u = step_size * m_hat / denom."""
    h = dict(lr=1e-2, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.5)
    rng = np.random.default_rng(8)
    n = 50000
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    tp, _, _ = _torch_adamw(p0, [g], h)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    ora.adamw(p, g, m, v, ora.hparams(step=1, **h))
    gd = g.astype(np.float64)
    u = h["lr"] * gd / (np.abs(gd) + h["eps"])
    diff = p.astype(np.float64) - tp.astype(np.float64)
    expected = h["lr"] * h["weight_decay"] * u
    assert np.abs(expected).min() > 1e3 * _ulp(p0).max()  # the effect is visible
    _close(diff, expected, 0, abs_tol=4 * _ulp(p0).max())


def test_zero_padding_stays_positive_zero(ora):
    for h in HP_SETS:
        for t in (1, 2, 1000):
            z = [np.zeros(16384, np.float32) for _ in range(4)]
            ora.adamw(z[0], z[1], z[2], z[3], ora.hparams(step=t, **h))
            for a in (z[0], z[2], z[3]):
                assert (a.view(np.uint32) == 0).all()


def test_second_moment_nonnegative(ora):
    rng = np.random.default_rng(9)
    n = 30000
    p = rng.normal(0, 0.02, n).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 6):
        g = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
        ora.adamw(p, g, m, v, ora.hparams(step=t))
        assert (v >= 0).all() and np.isfinite(p).all()
