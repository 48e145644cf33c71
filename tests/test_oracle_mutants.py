"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/oracle.c (a dropped term,
a wrong sign or index, a transposed operand, a wrong constant or rounding
rule), builds it into a throw-away library, points the oracle's ctypes
front at it and runs the fast pins.  At least one pin must fail for every
planted mistake.  The real oracle is never modified.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from tests import test_oracle_adamw as A
from tests import test_oracle_e4m3 as E
from tests import test_oracle_layout as L
from tests import test_oracle_plan as P
from tests import test_oracle_quant as Q
from tests import test_oracle_transpose as X

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "m uses beta1 for the gradient term": ("s->c1 * g", "s->b1 * g"),
    "v drops the gradient square": ("s->c2 * (g * g)", "s->c2 * g"),
    "denominator drops sqrt of bias correction 2": ("sqrtf(vv) / s->sbc2", "sqrtf(vv)"),
    "step size drops bias correction 1": ("(float)(hp->lr / (1.0 - pow(hp->beta1, t)))", "(float)hp->lr"),
    "eps inside the square root": ("sqrtf(vv) / s->sbc2 + s->eps", "sqrtf(vv + s->eps) / s->sbc2"),
    "update sign flipped": ("*p - s->step_size", "*p + s->step_size"),
    "decay applied to the old parameter": ("if (s->has_decay) pp = pp - s->decay * pp;",
                                           "if (s->has_decay) pp = pp - s->decay * *p;"),
    "beta2 swapped into the first moment": ("s.b1 = (float)hp->beta1;", "s.b1 = (float)hp->beta2;"),
    "E4M3 bias 8 (FNUZ-like)": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "ties round up": ("c = (k % 2 == 0) ? k : k + 1;", "c = k + 1;"),
    "saturates at the FNUZ maximum": ("if (a > 448.0) a = 448.0;", "if (a > 240.0) a = 240.0;"),
    "sign bit dropped": ("signbit(y) ? (c | 0x80) : c", "c"),
    "scale uses 240": (": amax / 448.0f;", ": amax / 240.0f;"),
    "quotient multiplies by the scale": ("float y = x[k] / s;", "float y = x[k] * s;"),
    "zero tile scale 0": ("scale_inv[t] = 1.0f;", "scale_inv[t] = 0.0f;"),
    "midpoint window absolute": ("return fabs(a - mid) <= rel * mid;", "return fabs(a - mid) <= rel;"),
    "power-of-two scale floor at the smallest normal": ("    int T = -149;\n    while (ldexp(448.0, T) < (double)amax) ++T;",
                                                         "    int T = -126;\n    while (ldexp(448.0, T) < (double)amax) ++T;"),
    "transpose: groups keep the tile scale": ("double g = amax == 0.0 ? 1.0 : pow2_scale_d(amax);",
                                              "double g = amax == 0.0 ? 1.0 : tile_scale;"),
    "underflowed scale kept at 0": ("if (s == 0.0f) s = (float)ldexp(1.0, -149);", ""),
    "amax ignores negatives": ("if (fabsf(x[k]) > amax) amax = fabsf(x[k]);", "if (x[k] > amax) amax = x[k];"),
    "quota rounds down": ("int64_t q = ceil_div(T, D);", "int64_t q = T / D + (T % D != 0 && T < D);"),
    "param-wise: smallest weight first": ("if (size > pick_size) { pick = p; pick_size = size; }",
                                          "if (pick < 0 || size < pick_size) { pick = p; pick_size = size; }"),
    "param-wise: fullest bucket": ("if (bucket_elems[b] < bucket_elems[best]) best = b;",
                                   "if (bucket_elems[b] > bucket_elems[best]) best = b;"),
    "power-of-two scale rounds down": ("while (ldexp(448.0, T) < (double)amax) ++T;",
                                       "while (ldexp(448.0, T + 1) < (double)amax) ++T;"),
    "transpose: group scale one step too small": ("while (ldexp(448.0, T) < amax) ++T;",
                                                  "while (ldexp(448.0, T + 1) < amax) ++T;"),
    "transpose: W^T row stride W": ("dst_t[p][out_row * H + ORA_TILE_DIM * i + r] = code;",
                                    "dst_t[p][out_row * W + ORA_TILE_DIM * i + r] = code;"),
    "valid rows from W": ("row[4] = (H - ORA_TILE_DIM * i) < ORA_TILE_DIM ? H - ORA_TILE_DIM * i : ORA_TILE_DIM;",
                          "row[4] = (W - ORA_TILE_DIM * i) < ORA_TILE_DIM ? W - ORA_TILE_DIM * i : ORA_TILE_DIM;"),
    "fold transposes the tile": ("tile[a * ORA_TILE_DIM + b] =", "tile[b * ORA_TILE_DIM + a] ="),
    "fold pads with the edge value": ("(r < H && c < W) ? src[(e * H + r) * W + c] : 0.0f",
                                      "src[(e * H + (r < H ? r : H - 1)) * W + (c < W ? c : W - 1)]"),
    "scale grid strided by hb": ("dst_scale[p][(e * hb + i) * wb + j]", "dst_scale[p][(e * hb + j) * hb + i]"),
    "unfold expert stride uses W": ("(e * H + ORA_TILE_DIM * i + a) * W", "(e * W + ORA_TILE_DIM * i + a) * W"),
    "fold reads one row low": ("src[(e * H + r) * W + c]", "src[(e * H + r - (r > 0)) * W + c]"),
}


def _pins():
    o = oracle
    pins = [lambda: E.test_decode_golden(o), lambda: E.test_encode_golden(o),
            lambda: E.test_value_table_structure(o), lambda: E.test_near_midpoint_flags(o)]
    for k in range(len(A.HP_SETS)):
        for gs in (1e-3, 1e-8, 3.0):
            pins.append(lambda k=k, gs=gs: A.test_first_step_closed_form(o, k, gs))
        for t in (2, 11, 1000):
            pins.append(lambda k=k, t=t: A.test_warm_state_closed_form(o, t, k))
    pins += [lambda: A.test_matches_torch_adamw_without_decay(o),
             lambda: A.test_weight_decay_placement_vs_torch(o),
             lambda: A.test_zero_padding_stays_positive_zero(o)]
    for kind in ("normal", "heavy", "wide"):
        pins.append(lambda kind=kind: Q.test_invariants(o, kind))
        pins.append(lambda kind=kind: Q.test_same_layout_requant_is_idempotent(o, kind))
    pins += [lambda: Q.test_exact_grid_tile(o), lambda: Q.test_block_quantize_multiply_form(o),
             lambda: Q.test_zero_tile_guard_and_padding(o), lambda: Q.test_pow2_scale_edges(o),
             lambda: Q.test_scale_underflow_floor(o)]
    for kind in ("normal", "heavy", "wide"):
        pins.append(lambda kind=kind: Q.test_pow2_invariants(o, kind))
    pins += [lambda s=s: P.test_brute_force_ownership(o, s) for s in range(4)]
    pins += [lambda: P.test_toy_walkthrough(o), lambda: P.test_workload_counts(o),
             lambda: P.test_more_ranks_than_tiles(o), lambda: P.test_paramwise_graham_worst_case(o),
             lambda: P.test_paramwise_too_few_weights(o)]
    pins += [lambda s=s: P.test_paramwise_brute_force(o, s) for s in range(10)]
    pins += [lambda sh=sh: L.test_pack_matches_im2col(o, sh) for sh in L.SHAPES]
    pins += [lambda sh=sh: L.test_unpack_matches_col2im(o, sh) for sh in L.SHAPES]
    pins.append(lambda: L.test_round_trip_multi_param_multi_rank(o))
    for case in range(len(X.SHAPES)):
        pins.append(lambda case=case: X.test_transpose_is_lossless(o, case))
        pins.append(lambda case=case: X.test_transpose_matches_torch_route(o, case))
    return pins


def _run_pins(lib_path):
    """Body of a child process: exit 0 if every pin passes on lib_path."""
    oracle._lib = None
    oracle.LIB_PATH = lib_path
    for pin in _pins():
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:
            sys.exit(1)
    sys.exit(0)


def _build(src_text, d):
    c = os.path.join(d, "oracle.c")
    with open(c, "w") as f:
        f.write(src_text)
    with open(os.path.join(d, "oracle.h"), "w") as f:
        f.write(open(os.path.join(os.path.dirname(SRC), "oracle.h")).read())
    lib = os.path.join(d, "liboracle_variant.so")
    subprocess.check_call(["gcc", "-O2", "-std=gnu99", "-fPIC", "-shared", "-ffp-contract=off",
                           c, "-o", lib, "-lm"])
    return lib


def _caught(lib_path):
    """True when some pin fails on lib_path -- or the planted mistake crashes
    the process (an out-of-bounds index), hence a fresh child process."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, OMP_NUM_THREADS="1", PYTHONFAULTHANDLER="")
    code = f"from tests.test_oracle_mutants import _run_pins; _run_pins({lib_path!r})"
    try:
        r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, timeout=600,
                           stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    except subprocess.TimeoutExpired:
        return True
    return r.returncode != 0


def test_unmutated_copy_passes_all_pins(tmp_path):
    assert not _caught(_build(open(SRC).read(), str(tmp_path)))


@pytest.mark.slow
def test_planted_mistakes_are_caught(tmp_path):
    src = open(SRC).read()
    libs = {}
    for k, (name, (before, after)) in enumerate(sorted(MUTANTS.items())):
        assert src.count(before) == 1, f"mutation anchor not unique: {before!r}"
        d = tmp_path / f"m{k}"
        d.mkdir()
        libs[name] = _build(src.replace(before, after), str(d))
    with ThreadPoolExecutor(max_workers=max(1, (os.cpu_count() or 2) - 1)) as ex:
        caught = dict(zip(libs, ex.map(_caught, libs.values())))
    survivors = [n for n, c in caught.items() if not c]
    assert not survivors, survivors
