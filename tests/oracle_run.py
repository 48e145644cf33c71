"""The oracle's side of a parity check: regenerate one slot's inputs on the
host from the seeded generator, fold them with the oracle, and run the
workload's steps through the oracle.  Test infrastructure only."""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

import oracle
import synth
from synth import workloads as WL

TILE_ELEMS = oracle.TILE_ELEMS


def _fold_rect(w, tensor, p, e, i, j, vr, vc, step=0):
    r = w.recipe(tensor, p, step)
    rect = synth.fill_rect_host(r, e, 128 * i, vr, 128 * j, vc)
    return oracle.fold_tile(np.ascontiguousarray(rect.reshape(1, vr, vc)), 0, 0, 0)


def oracle_slot(w, row, steps=None, rel=1e-6, pow2=False):
    """Final master/m/v tile, codes, scale_inv and midpoint flags of the slot
    whose oracle plan row is `row` = (p, e, i, j, vr, vc)."""
    p, e, i, j, vr, vc = (int(x) for x in row)
    z = np.zeros(TILE_ELEMS, dtype=np.float32)
    if p < 0:
        master, m, v = z.copy(), z.copy(), z.copy()
        grads = {t: z.copy() for t in (steps or w.steps)}
    else:
        master = _fold_rect(w, WL.MASTER, p, e, i, j, vr, vc)
        m = _fold_rect(w, WL.MOM1, p, e, i, j, vr, vc)
        v = _fold_rect(w, WL.MOM2, p, e, i, j, vr, vc)
        grads = {t: _fold_rect(w, WL.GRAD, p, e, i, j, vr, vc, t) for t in (steps or w.steps)}
    out = None
    for t in (steps or w.steps):
        codes, scale, near = oracle.step(master, grads[t], m, v,
                                         oracle.hparams(step=t, **WL.HP), rel, pow2)
        out = (codes, scale, near)
    return dict(master=master, m=m, v=v, codes=out[0], scale_inv=out[1][0], near=out[2])


def oracle_slots(w, slots, steps=None, rel=1e-6, threads=None, pow2=False):
    q, owned, table = oracle.plan(w.dims, w.D, w.rank)
    threads = threads or min(16, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(lambda s: oracle_slot(w, table[s], steps, rel, pow2), slots))
    keys = ("master", "m", "v", "codes", "near")
    out = {k: np.stack([r[k] for r in res]) for k in keys}
    out["scale_inv"] = np.array([r["scale_inv"] for r in res], dtype=np.float32)
    out["table"] = table[np.asarray(slots, dtype=np.int64)]
    return out


def sample_slots(w, n_random=96, seed=0):
    """First, last, padding and edge slots, weight boundaries, a few zero
    tiles where the workload has them, and a seeded random sample."""
    q, owned, table = oracle.plan(w.dims, w.D, w.rank)
    pick = {0, max(0, owned - 1), q - 1}
    for s in range(1, owned):
        if table[s][0] != table[s - 1][0]:
            pick.update((s - 1, s))
        if len(pick) > 60:
            break
    edge = [s for s in range(owned) if table[s][4] < 128 or table[s][5] < 128]
    pick.update(edge[:8] + edge[-8:])
    if w.zero_tile_prob > 0:
        zeros = []
        for s in range(owned):
            p, e, i, j = (int(x) for x in table[s][:4])
            E, H, W = w.dims[p]
            hb, wb = -(-H // 128), -(-W // 128)
            if synth.lib().synth_uniform(w._zero_key(p), (e * hb + i) * wb + j) < w.zero_tile_prob:
                zeros.append(s)
            if len(zeros) >= 8:
                break
        pick.update(zeros)
    rng = np.random.default_rng(seed)
    pick.update(int(x) for x in rng.integers(0, q, size=min(n_random, q)))
    return sorted(pick)
