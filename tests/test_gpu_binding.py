"""The binding's marshalling on the GPU: master / m / v as contiguous
tensors or as (tiles, 16384) views of one (q, 3, 16384) tensor (the stride
each call passes in bfz_step_options.state_stride is the views' row
stride), per-weight tensors checked against the plan's shapes, and
inconsistent arguments refused before any kernel runs."""
import sys

import numpy as np
import pytest
import torch

import blockwise_fp8_zero_amd as bfz

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _say(*a):
    print("[gpu-binding]", *a, flush=True)
    sys.stdout.flush()


def _bufs(q):
    f32 = dict(dtype=torch.float32, device="cuda")
    g = torch.randn(q * 16384, **f32) * 1e-3
    codes = torch.empty(q * 16384, dtype=torch.uint8, device="cuda")
    sc = torch.empty(q, **f32)
    return g, codes, sc


def test_mismatched_state_strides_are_refused():
    q = 3
    _say("state-stride checks, q =", q)
    g, codes, sc = _bufs(q)
    state = torch.zeros(q, 3, 16384, dtype=torch.float32, device="cuda")
    flat = torch.zeros(q * 16384, dtype=torch.float32, device="cuda")
    hp = bfz.AdamW(step=1, **HP)
    with pytest.raises(ValueError, match="different tile strides"):
        bfz.adamw_fp8_step(state[:, 0], g, flat, state[:, 2], codes, sc, hp)
    gappy = torch.zeros(q, 2 * 16384, dtype=torch.float32, device="cuda")[:, ::2]
    with pytest.raises(TypeError):  # (q, 16384) but its elements are not contiguous within a tile
        bfz.adamw_fp8_step(gappy, g, state[:, 1], state[:, 2], codes, sc, hp)
    with pytest.raises(ValueError, match="tiles"):
        bfz.adamw_fp8_step(state[:2, 0], g, state[:2, 1], state[:2, 2], codes, sc, hp, n_tiles=3)
    torch.cuda.synchronize()
    assert not state.any()  # nothing ran


def test_caller_hp_is_not_modified_and_layouts_agree():
    """The same step through contiguous arrays (adamw_fp8_step) and through
    interleaved views (adamw_fp8_step_ex with state_stride 49152) gives
    bit-identical results; the caller's AdamW struct is left as it was."""
    q = 5
    _say("layout agreement through the binding, q =", q)
    torch.manual_seed(3)
    g, codes_a, sc_a = _bufs(q)
    codes_b = torch.empty_like(codes_a)
    sc_b = torch.empty_like(sc_a)
    p0 = torch.randn(q, 16384, device="cuda") * 0.02
    m0 = torch.randn(q, 16384, device="cuda") * 1e-4
    v0 = torch.rand(q, 16384, device="cuda") * 1e-6
    sep = [x.clone().reshape(-1) for x in (p0, m0, v0)]
    state = torch.stack([p0, m0, v0], dim=1).contiguous()
    hp = bfz.AdamW(step=7, **HP)
    bfz.adamw_fp8_step(*sep[:1], g, *sep[1:], codes_a, sc_a, hp)
    bfz.adamw_fp8_step(state[:, 0], g, state[:, 1], state[:, 2], codes_b, sc_b, hp)
    torch.cuda.synchronize()
    assert bytes(hp) == bytes(bfz.AdamW(step=7, **HP))
    for k in range(3):
        assert torch.equal(sep[k].view(torch.int32), state[:, k].reshape(-1).view(torch.int32)), k
    assert torch.equal(codes_a, codes_b) and torch.equal(sc_a, sc_b)
    assert not np.array_equal(sep[0].cpu().numpy(), p0.reshape(-1).cpu().numpy())  # it did step


def test_single_tile_and_empty_views():
    """q = 1: a (1, 16384) view has no stride of its own and is accepted
    next to contiguous tensors; n_tiles = 0 is a no-op."""
    _say("single-tile views and n_tiles = 0")
    g, codes, sc = _bufs(1)
    state = torch.zeros(1, 3, 16384, dtype=torch.float32, device="cuda")
    state[:, 0] = 0.5
    flat = torch.zeros(16384, dtype=torch.float32, device="cuda")
    hp = bfz.AdamW(step=1, **HP)
    bfz.adamw_fp8_step(state[:, 0], g, flat, state[:, 2], codes, sc, hp)
    torch.cuda.synchronize()
    assert float(sc[0]) > 0 and flat.abs().sum() > 0
    before = state.clone()
    bfz.adamw_fp8_step(state[:, 0], g, state[:, 1], state[:, 2], codes, sc, hp, n_tiles=0)
    torch.cuda.synchronize()
    assert torch.equal(before, state)


def test_pack_shard_strided_flat_buffer_equals_views():
    """pack_shard_strided into a flat buffer at stride 49152 gives, bit for
    bit, the tiles pack_shard writes into a (q, 16384) view of the same
    layout and into a contiguous shard; the gaps are not written."""
    dims = [(1, 300, 200), (2, 129, 257)]
    plan = bfz.Plan(dims, 2, 1)
    q = plan.shard_tiles
    _say("pack_shard_strided, dims", dims, "q =", q)
    torch.manual_seed(5)
    src = [torch.randn(E * H * W, device="cuda") for E, H, W in dims]
    flat = torch.full((q * 49152,), -1.0, device="cuda")
    bfz.pack_shard_strided(plan, src, flat, 49152)
    view = torch.full((q, 3, 16384), -1.0, device="cuda")
    bfz.pack_shard(plan, src, view[:, 1])
    ref = torch.empty(q * 16384, device="cuda")
    bfz.pack_shard(plan, src, ref)
    torch.cuda.synchronize()
    tiles = flat.view(q, 3, 16384)[:, 0]
    assert torch.equal(tiles.reshape(-1).view(torch.int32), ref.view(torch.int32))
    assert torch.equal(view[:, 1].reshape(-1).view(torch.int32), ref.view(torch.int32))
    assert (flat.view(q, 3, 16384)[:, 1:] == -1.0).all() and (view[:, 0::2] == -1.0).all()
    with pytest.raises(ValueError):  # too short for q tiles at this stride
        bfz.pack_shard_strided(plan, src, flat[: (q - 1) * 49152], 49152)



@pytest.mark.parametrize("mode", ["unfused", "fused", "fused_unpack"])
def test_gapped_state_stride(mode):
    """A state layout with gaps -- four tile slots per block, the fourth
    unused (state_stride 65536) -- through every step route on ragged
    weights that span several tiles: bit-identical to three separate
    arrays, and the gap slots are never written."""
    from synth import workloads as WL
    from bench_workload import GpuWorkload
    w = WL.ragged()
    w.dims = w.dims[:6]
    _say("gapped state stride 65536, 6 ragged matrices, mode", mode)
    ref = GpuWorkload(w, mode=mode, layout="separate")
    gap = GpuWorkload(w, mode=mode, layout="separate")
    q = gap.q
    block = torch.full((q, 4, 16384), 7.0, dtype=torch.float32, device="cuda")
    gap.master, gap.m, gap.v = block[:, 0], block[:, 1], block[:, 2]
    for g in (ref, gap):
        g.load_state()
        g.run_steps()
    torch.cuda.synchronize()
    a = ref.tiles(list(range(q)))
    b = gap.tiles(list(range(q)))
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    assert (block[:, 3] == 7.0).all()


def test_undersized_per_weight_tensors_are_refused():
    """Each per-weight tensor must hold its whole row-major weight (or scale
    grid): the kernels address it through the plan's table, so a smaller one
    would be read or written out of bounds.  Refused with ValueError before
    any launch, for every entry point that takes per-weight tensors."""
    dims = [(2, 200, 300), (1, 129, 130)]
    plan = bfz.Plan(dims, 1, 0)
    q = plan.shard_tiles
    _say("per-weight size checks, dims", dims, "q =", q)
    f32 = dict(dtype=torch.float32, device="cuda")
    u8 = dict(dtype=torch.uint8, device="cuda")
    full = [E * H * W for E, H, W in dims]
    grid = [E * -(-H // 128) * -(-W // 128) for E, H, W in dims]
    tgrid = [E * W * -(-H // 128) for E, H, W in dims]
    grads = [torch.zeros(n, **f32) for n in full]
    short = [torch.zeros(200 * 300, **f32), grads[1]]   # one expert of two
    st = [torch.zeros(q * 16384, **f32) for _ in range(3)]
    codes = torch.zeros(q * 16384, **u8)
    sc = torch.zeros(q, **f32)
    d8 = [torch.zeros(n, **u8) for n in full]
    dsc = [torch.zeros(n, **f32) for n in grid]
    dt = [torch.zeros(n, **u8) for n in full]
    dts = [torch.zeros(n, **f32) for n in tgrid]
    hp = bfz.AdamW(step=1, **HP)
    with pytest.raises(ValueError, match=r"srcs\[0\]"):
        bfz.pack_shard(plan, short, st[0])
    with pytest.raises(ValueError, match=r"grads\[0\]"):
        bfz.fold_adamw_fp8_step(plan, short, *st, codes, sc, hp)
    with pytest.raises(ValueError, match=r"dst_fp8\[1\]"):
        bfz.unpack_fp8(plan, codes, sc, [d8[0], d8[1][:-1]], dsc)
    with pytest.raises(ValueError, match=r"dst_scale\[0\]"):   # a grid sized W / 128, not E hb wb
        bfz.fold_adamw_fp8_step_unpack(plan, grads, *st, codes, sc, d8,
                                       [torch.zeros(3, **f32), dsc[1]], hp)
    with pytest.raises(ValueError, match=r"dst_t_scale\[0\]"):
        bfz.fold_adamw_fp8_step_unpack_t(plan, grads, *st, codes, sc, d8, dsc, dt,
                                         [dsc[0], dts[1]], hp)
    with pytest.raises(ValueError, match=r"dst_t\[1\]"):
        bfz.transpose_pow2(plan, codes, sc, [dt[0], dt[1][:100]], dts)
    with pytest.raises(ValueError, match="3 tensors for 2 weights"):
        bfz.pack_shard(plan, grads + [grads[0]], st[0])
    torch.cuda.synchronize()
    assert not any(x.any() for x in st + d8 + dsc + dt + dts) and not codes.any()  # nothing ran


def test_plain_call_sequence_through_the_raw_abi():
    """The boundary's basic sequence called straight through ctypes with a
    caller-defined six-field hyper-parameter struct (48 bytes, no options):
    bfz_plan_create (which copies the table to the device; no
    bfz_plan_upload call), pack_shard of master / m / v / gradient into three
    separate tile-major arrays, adamw_fp8_step, unpack_fp8 -- bit-exact
    with the oracle on every slot, row-major output included."""
    import ctypes as C

    import oracle
    from synth import workloads as WL
    from tests.compare import compare
    from tests.oracle_run import oracle_slots

    class Hyper(C.Structure):  # the caller's own copy of bfz_adamw
        _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                    ("eps", C.c_double), ("weight_decay", C.c_double), ("step", C.c_int64)]

    assert C.sizeof(Hyper) == 48
    w = WL.tiny()
    _say("raw ABI sequence on", w.name, w.dims, "steps", w.steps)
    L = C.CDLL(bfz.LIB_PATH)
    P = C.c_void_p
    L.bfz_plan_create.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, C.POINTER(P)]
    L.bfz_plan_shard_tiles.restype = C.c_int64
    L.bfz_plan_shard_tiles.argtypes = [P]
    L.bfz_plan_destroy.argtypes = [P]
    L.bfz_plan_destroy.restype = None
    L.pack_shard.argtypes = [P, P, P, P]
    L.adamw_fp8_step.argtypes = [P, P, P, P, P, P, C.c_int64, C.POINTER(Hyper), P]
    L.unpack_fp8.argtypes = [P, P, P, P, P, P]
    L.bfz_last_error.restype = C.c_char_p
    dims = (C.c_int64 * 3)(*w.dims[0])
    plan = P()
    assert L.bfz_plan_create(C.cast(dims, P), 1, w.D, w.rank, C.byref(plan)) == 0, L.bfz_last_error()
    q = L.bfz_plan_shard_tiles(plan)
    E, H, W = w.dims[0]
    import synth
    f32 = dict(dtype=torch.float32, device="cuda")

    def rowmajor(tensor, step=0):
        b = torch.empty(E * H * W, **f32)
        synth.fill_device(w.recipe(tensor, 0, step), b, 0, E * H * W)
        return b

    stream = P(torch.cuda.current_stream().cuda_stream)
    tiles = {k: torch.empty(q * 16384, **f32) for k in ("p", "m", "v", "g")}
    for k, tensor in (("p", WL.MASTER), ("m", WL.MOM1), ("v", WL.MOM2)):
        src = rowmajor(tensor)
        arr = (P * 1)(src.data_ptr())
        assert L.pack_shard(plan, C.cast(arr, P), P(tiles[k].data_ptr()), stream) == 0, L.bfz_last_error()
        torch.cuda.synchronize()
    codes = torch.empty(q * 16384, dtype=torch.uint8, device="cuda")
    sc = torch.empty(q, **f32)
    for t in w.steps:
        g = rowmajor(WL.GRAD, t)
        arr = (P * 1)(g.data_ptr())
        assert L.pack_shard(plan, C.cast(arr, P), P(tiles["g"].data_ptr()), stream) == 0
        hp = Hyper(step=t, **WL.HP)
        assert L.adamw_fp8_step(P(tiles["p"].data_ptr()), P(tiles["g"].data_ptr()), P(tiles["m"].data_ptr()),
                                P(tiles["v"].data_ptr()), P(codes.data_ptr()), P(sc.data_ptr()), q,
                                C.byref(hp), stream) == 0, L.bfz_last_error()
        torch.cuda.synchronize()
    fp8 = torch.zeros(E * H * W, dtype=torch.uint8, device="cuda")
    grid = torch.zeros(E * -(-H // 128) * -(-W // 128), **f32)
    a8, asc = (P * 1)(fp8.data_ptr()), (P * 1)(grid.data_ptr())
    assert L.unpack_fp8(plan, P(codes.data_ptr()), P(sc.data_ptr()), C.cast(a8, P), C.cast(asc, P),
                        stream) == 0, L.bfz_last_error()
    torch.cuda.synchronize()
    slots = list(range(q))
    ora = oracle_slots(w, slots)
    gpu = dict(master=tiles["p"].view(q, -1).cpu().numpy(), m=tiles["m"].view(q, -1).cpu().numpy(),
               v=tiles["v"].view(q, -1).cpu().numpy(), codes=codes.view(q, -1).cpu().numpy(),
               scale_inv=sc.cpu().numpy())
    rep = compare(gpu, ora)
    _say("raw ABI sequence:", {k: v for k, v in rep.items() if k != "fail"})
    assert rep["ok"] and rep["exact"], rep["fail"]
    _, _, table = oracle.plan(w.dims, w.D, w.rank)
    o8 = np.zeros((E, H, W), dtype=np.uint8)
    osc = np.zeros((E, -(-H // 128), -(-W // 128)), dtype=np.float32)
    oracle.unpack(w.dims, ora["codes"].reshape(-1), ora["scale_inv"], table, [o8], [osc])
    assert np.array_equal(fp8.cpu().numpy(), o8.reshape(-1))
    assert np.array_equal(grid.cpu().numpy(), osc.reshape(-1))
    L.bfz_plan_destroy(plan)
