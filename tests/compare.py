"""Element-wise comparison of the HIP path against the oracle.

The bar: FP32 master, m and v within |gpu - ora| <= 1e-9 + 1e-6 |ora|;
scale_inv within rel 1e-6; E4M3 codes equal, except where the oracle's
quotient p / scale_inv sits within rel 1e-6 of a rounding midpoint -- there
the code may be either neighbour; such elements are counted and reported.
Bit-exact agreement is counted separately (the kernels evaluate the same
binary32 operations in the same order as the oracle, so it is expected).
"""
import numpy as np

import oracle

REL, ABS = 1e-6, 1e-9

_DEC = None


def _dec():
    global _DEC
    if _DEC is None:
        _DEC = np.array([oracle.e4m3_decode(c) for c in range(256)])
    return _DEC


def compare(gpu: dict, ora: dict):
    """Returns a report dict; report['ok'] says whether every element meets the bar above."""
    rep = {"ok": True, "fail": []}
    for k in ("master", "m", "v"):
        g = np.asarray(gpu[k], dtype=np.float64).reshape(-1)
        o = np.asarray(ora[k], dtype=np.float64).reshape(-1)
        bad = np.abs(g - o) > ABS + REL * np.abs(o)
        rep[f"{k}_bad"] = int(bad.sum())
        rep[f"{k}_exact"] = bool(np.array_equal(np.asarray(gpu[k]).view(np.uint32).reshape(-1),
                                                np.asarray(ora[k]).view(np.uint32).reshape(-1)))
        if bad.any():
            rep["ok"] = False
            rep["fail"].append(f"{k}: {int(bad.sum())} elements out of tolerance")
    gs = np.asarray(gpu["scale_inv"], dtype=np.float64).reshape(-1)
    os_ = np.asarray(ora["scale_inv"], dtype=np.float64).reshape(-1)
    bad = np.abs(gs - os_) > REL * np.abs(os_)
    rep["scale_bad"] = int(bad.sum())
    rep["scale_exact"] = bool(np.array_equal(gs, os_))
    if bad.any():
        rep["ok"] = False
        rep["fail"].append(f"scale_inv: {int(bad.sum())} tiles out of tolerance")
    gc = np.asarray(gpu["codes"]).reshape(-1)
    oc = np.asarray(ora["codes"]).reshape(-1)
    near = np.asarray(ora["near"]).reshape(-1).astype(bool)
    diff = gc != oc
    rep["codes_mismatch"] = int(diff.sum())
    rep["codes_mismatch_near_midpoint"] = int((diff & near).sum())
    rep["near_midpoint_elems"] = int(near.sum())
    hard = diff & ~near
    if hard.any():
        rep["ok"] = False
        rep["fail"].append(f"codes: {int(hard.sum())} mismatches away from midpoints")
    soft = diff & near
    if soft.any():  # must be a neighbouring value of the same sign
        dec = _dec()
        g, o = dec[gc[soft]], dec[oc[soft]]
        vals = np.unique(np.abs(dec[np.isfinite(dec)]))
        gi = np.searchsorted(vals, np.abs(g))
        oi = np.searchsorted(vals, np.abs(o))
        far = (np.abs(gi - oi) > 1) | ((np.signbit(g) != np.signbit(o)) & (g != 0) & (o != 0))
        if far.any():
            rep["ok"] = False
            rep["fail"].append(f"codes: {int(far.sum())} midpoint cases not a neighbour")
    rep["codes_exact"] = not diff.any()
    rep["exact"] = all(rep[f"{k}_exact"] for k in ("master", "m", "v")) and rep["scale_exact"] \
        and rep["codes_exact"]
    return rep
