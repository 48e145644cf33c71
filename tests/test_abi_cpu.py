"""The C ABI on the CPU: the library loads, exports every function
include/bfz.h declares, plans exactly like the oracle, and rejects bad
arguments before touching any GPU.  No compute call runs here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import blockwise_fp8_zero_amd as bfz
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "bfz.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)
    return sorted({n for n in names if n not in ("if", "defined")})


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"pack_shard", "adamw_fp8_step", "unpack_fp8", "bfz_plan_create",
            "bfz_last_error"} <= set(names)
    L = bfz.lib()
    for n in names:
        assert hasattr(L, n), n


def test_plan_matches_oracle_plan():
    rng = np.random.default_rng(0)
    for trial in range(40):
        dims = [(int(rng.integers(1, 4)), int(rng.integers(1, 900)), int(rng.integers(1, 900)))
                for _ in range(int(rng.integers(1, 7)))]
        D = int(rng.integers(1, 10))
        for r in range(D):
            q, owned, table = oracle.plan(dims, D, r)
            p = bfz.Plan(dims, D, r)
            assert (p.shard_tiles, p.owned_tiles, p.total_tiles) == (q, owned, oracle.total_tiles(dims))
            assert np.array_equal(p.table(), table)
            if q:
                assert p.tile(q - 1) == tuple(table[q - 1])
            p.close()


def test_plan_of_the_workloads():
    from synth import workloads as WL
    for f in WL.ALL:
        w = f()
        q, owned, table = oracle.plan(w.dims, w.D, w.rank)
        p = bfz.Plan(w.dims, w.D, w.rank)
        assert p.shard_tiles == q and p.owned_tiles == owned
        assert np.array_equal(p.table(), table), w.name


def test_paramwise_split_matches_oracle():
    from synth import workloads as WL
    rng = np.random.default_rng(3)
    cases = [([(int(rng.integers(1, 3)), int(rng.integers(1, 3000)), int(rng.integers(1, 3000)))
               for _ in range(int(rng.integers(1, 40)))], int(rng.integers(1, 17))) for _ in range(60)]
    cases += [([(1, 5, 5)] * 7, 3), ([(2, 4, 4), (1, 8, 4), (1, 4, 8)], 2)]  # size ties
    cases += [(f().dims, f().D) for f in WL.ALL]
    for dims, D in cases:
        a = bfz.paramwise_split(dims, D)
        b = oracle.paramwise_split(dims, D)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    with pytest.raises(bfz.BfzError):
        bfz.paramwise_split([(1, 0, 3)], 2)
    with pytest.raises(bfz.BfzError):
        bfz.paramwise_split([(1, 2, 3)], 0)
    # each weight is within bounds, their sum (2^63 elements) is not
    with pytest.raises(bfz.BfzError):
        bfz.paramwise_split([(1, 2 ** 31, 2 ** 31)] * 2, 2)
    bop, be = bfz.paramwise_split([(1, 2 ** 31, 2 ** 30)] * 2, 2)
    assert list(be) == [2 ** 61, 2 ** 61]


@pytest.mark.parametrize("dims,D,rank", [
    ([(1, 10, 10)], 0, 0), ([(1, 10, 10)], 2, 2), ([(1, 10, 10)], 2, -1),
    ([(0, 10, 10)], 1, 0), ([(1, 10, -3)], 1, 0), ([(1, 2 ** 31, 5)], 1, 0), ([], 1, 0),
    ([(2 ** 20, 8192, 8192)], 4096, 0),  # 2^32 tiles: the scale-grid index would overflow
    # three weights of 2^31 - 4096 tiles each: a quota past 2^31 - 1 tiles per rank,
    # refused before any table is allocated
    ([(2 ** 19 - 1, 8192, 8192)] * 3, 1, 0), ([(2 ** 19 - 1, 8192, 8192)] * 3, 2, 1),
])
def test_plan_rejects_bad_arguments(dims, D, rank):
    with pytest.raises(bfz.BfzError) as e:
        bfz.Plan(dims, D, rank)
    assert e.value.code == bfz.BFZ_EINVAL
    assert bfz.lib().bfz_last_error()


def _call_step(ptrs, n_tiles=1, hp=None, opts=None):
    """adamw_fp8_step (opts None) or adamw_fp8_step_ex on fake pointers."""
    hp = hp or bfz.AdamW(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    args = [C.c_void_p(p) for p in ptrs]
    if opts is None:
        return bfz.lib().adamw_fp8_step(*args, n_tiles, C.byref(hp), None)
    return bfz.lib().adamw_fp8_step_ex(*args, n_tiles, C.byref(hp), C.byref(opts), None)


def test_struct_sizes_match_the_header():
    """bfz_adamw is the six-field, 48-byte struct every step call reads;
    the options live in the 16-byte bfz_step_options."""
    assert C.sizeof(bfz.AdamW) == 48 and C.sizeof(bfz.StepOptions) == 16
    text = open(os.path.join(ROOT, "include", "bfz.h")).read()
    body = re.search(r"typedef struct \{([^}]*)\} bfz_adamw;", text).group(1)
    assert re.sub(r"\s+", " ", body).strip() == \
        "double lr, beta1, beta2, eps, weight_decay; int64_t step;"


def test_step_argument_errors_without_gpu():
    ok = [0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000]
    assert _call_step([0] + ok[1:]) == bfz.BFZ_EINVAL
    assert _call_step(ok, n_tiles=-1) == bfz.BFZ_EINVAL
    assert _call_step(ok, n_tiles=1 << 31) == bfz.BFZ_EINVAL
    assert _call_step(ok, n_tiles=(1 << 22)) == bfz.BFZ_EINVAL  # past 2^32 work-items
    for k in range(5):
        bad = list(ok)
        bad[k] += 4
        assert _call_step(bad) == bfz.BFZ_EALIGN
        assert "aligned" in bfz.lib().bfz_last_error().decode()
    bad = list(ok)
    bad[5] += 2
    assert _call_step(bad) == bfz.BFZ_EALIGN
    for field, val in (("beta1", 1.0), ("beta2", -0.1), ("eps", -1.0), ("eps", 0.0),
                       ("lr", float("nan")), ("step", 0), ("weight_decay", float("inf"))):
        hp = bfz.AdamW(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
        setattr(hp, field, val)
        assert _call_step(ok, hp=hp) == bfz.BFZ_EINVAL, field
        assert _call_step(ok, hp=hp, opts=bfz.StepOptions()) == bfz.BFZ_EINVAL, field
    assert "eps > 0" in bfz.lib().bfz_last_error().decode()
    assert _call_step(ok, opts=bfz.StepOptions(reserved=1)) == bfz.BFZ_EINVAL
    assert "reserved" in bfz.lib().bfz_last_error().decode()


@pytest.mark.parametrize("stride", [-16384, 1, 16383, 16386, 49150, (1 << 26) + 4, 1 << 40])
def test_bad_state_stride_is_rejected_without_gpu(stride):
    """state_stride: 0, or a multiple of 4 in [16384, 2^26] (tiles of
    master / m / v may not overlap and must stay 16-byte aligned)."""
    ok = [0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000]
    assert _call_step(ok, opts=bfz.StepOptions(state_stride=stride)) == bfz.BFZ_EINVAL
    assert "state_stride" in bfz.lib().bfz_last_error().decode()
    L = bfz.lib()
    p = bfz.Plan([(1, 256, 256)], 1, 0)
    src = (C.c_void_p * 1)(0x10000)
    assert L.pack_shard_strided(p.handle, C.cast(src, C.c_void_p), C.c_void_p(0x30000), stride,
                                None) == bfz.BFZ_EINVAL
    assert "dst_stride" in L.bfz_last_error().decode()
    p.close()


def test_good_state_stride_passes_the_checks():
    """Valid strides get past their check: pack_shard_strided stops at the
    plan (no device here, so no device table: BFZ_ESTATE), and a step whose
    only fault is beta1 = 1 reports that, not the stride."""
    L = bfz.lib()
    p = bfz.Plan([(1, 256, 256)], 1, 0)
    src = (C.c_void_p * 1)(0x10000)
    ok = [0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000]
    for stride in (0, 16384, 49152, 1 << 26):
        assert L.pack_shard_strided(p.handle, C.cast(src, C.c_void_p), C.c_void_p(0x30000),
                                    stride or 16384, None) == bfz.BFZ_ESTATE
        hp = bfz.AdamW(lr=1e-4, beta1=1.0, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
        assert _call_step(ok, hp=hp, opts=bfz.StepOptions(state_stride=stride)) == bfz.BFZ_EINVAL
        msg = L.bfz_last_error().decode()
        assert "beta" in msg and "state_stride" not in msg, msg
    p.close()


def test_pack_unpack_errors_without_gpu():
    L = bfz.lib()
    p = bfz.Plan([(1, 256, 256), (1, 128, 128)], 2, 0)
    src = (C.c_void_p * 2)(0x10000, 0x20000)
    # no HIP device in this container: the plan has no device table
    assert L.pack_shard(p.handle, C.cast(src, C.c_void_p), C.c_void_p(0x30000), None) == bfz.BFZ_ESTATE
    assert L.pack_shard(p.handle, None, C.c_void_p(0x30000), None) == bfz.BFZ_EINVAL
    assert L.pack_shard(None, C.cast(src, C.c_void_p), C.c_void_p(0x30000), None) == bfz.BFZ_EINVAL
    d8 = (C.c_void_p * 2)(0x10000, 0x20000)
    assert L.unpack_fp8(p.handle, C.c_void_p(0x40000), C.c_void_p(0x50000), C.cast(d8, C.c_void_p),
                        C.cast(d8, C.c_void_p), None) == bfz.BFZ_ESTATE
    hp = bfz.AdamW(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    st = [C.c_void_p(x) for x in (0x40000, 0x50000, 0x60000, 0x70000, 0x80000)]
    assert L.fold_adamw_fp8_step(p.handle, C.cast(src, C.c_void_p), *st, C.byref(hp), None,
                                 None) == bfz.BFZ_ESTATE
    assert L.fold_adamw_fp8_step(p.handle, None, *st, C.byref(hp), None, None) == bfz.BFZ_EINVAL
    assert L.fold_adamw_fp8_step(None, C.cast(src, C.c_void_p), *st, C.byref(hp), None,
                                 None) == bfz.BFZ_EINVAL
    assert "no device table" in (L.pack_shard(p.handle, C.cast(src, C.c_void_p), C.c_void_p(0x30000),
                                              None) and L.bfz_last_error().decode())
    assert L.bfz_e4m3_encode(None, C.c_void_p(0x10), 5, None) == bfz.BFZ_EINVAL
    assert L.bfz_e4m3_encode(C.c_void_p(0x10), C.c_void_p(0x10), -1, None) == bfz.BFZ_EINVAL
    assert L.bfz_plan_tile(p.handle, 99, C.cast((C.c_int64 * 6)(), C.c_void_p)) == bfz.BFZ_EINVAL
    p.close()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libbfz.so every call raises: there is no non-HIP fallback."""
    import blockwise_fp8_zero_amd as bfz
    monkeypatch.setattr(bfz, "LIB_PATH", str(tmp_path / "libbfz.so"))
    monkeypatch.setattr(bfz, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        bfz.Plan([(1, 128, 128)], 1, 0)
