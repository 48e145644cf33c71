"""Python binding of libbfz.so, the block-wise FP8 ZeRO-1 shard step.

Argument marshalling only: every step of the path runs in the library's HIP
kernels (see include/bfz.h for the operations, layouts and error codes).
PyTorch supplies device memory and the stream; the functions take torch
tensors, check dtype / device / size, and pass raw pointers plus
torch.cuda.current_stream() to the C ABI.  If the library is not built,
importing works but every call raises -- there is no fallback path.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbfz.so")
TILE = 128
TILE_ELEMS = TILE * TILE
# the interleaved state layout (BFZ_STATE_STRIDE_INTERLEAVED): one
# [master | m | v] block per tile and a 4 KiB gap; with
# state = torch.zeros(q, STATE_STRIDE), pass state[:, :16384],
# state[:, 16384:32768] and state[:, 32768:49152] as master, m and v
STATE_STRIDE = 50176

BFZ_OK, BFZ_EINVAL, BFZ_EALIGN, BFZ_EHIP, BFZ_ESTATE = 0, -1, -2, -3, -4


class BfzError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"bfz error {code}: {msg}")
        self.code = code


class AdamW(C.Structure):
    """bfz_adamw: the hyper-parameters of one step; step is the counter t >= 1."""
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("step", C.c_int64)]


class StepOptions(C.Structure):
    """bfz_step_options: power-of-two tile scales, and the tile stride of
    master / m / v (the step functions fill it in from the state tensors)."""
    _fields_ = [("scale_pow2", C.c_int32), ("reserved", C.c_int32), ("state_stride", C.c_int64)]


_lib = None


def lib():
    """The loaded libbfz.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build()); "
                               "this package has no non-HIP fallback")
        L = C.CDLL(LIB_PATH)
        P, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.bfz_plan_create.argtypes = [P, i32, i32, i32, C.POINTER(P)]
        L.bfz_plan_upload.argtypes = [P]
        L.bfz_plan_destroy.argtypes = [P]
        L.bfz_plan_destroy.restype = None
        for n in ("bfz_plan_shard_tiles", "bfz_plan_owned_tiles", "bfz_plan_total_tiles"):
            getattr(L, n).argtypes = [P]
            getattr(L, n).restype = i64
        L.bfz_plan_table.argtypes = [P, P]
        L.bfz_plan_tile.argtypes = [P, i64, P]
        L.bfz_paramwise_split.argtypes = [P, i32, i32, P, P]
        L.pack_shard.argtypes = [P, P, P, P]
        L.pack_shard_strided.argtypes = [P, P, P, i64, P]
        A, O = C.POINTER(AdamW), C.POINTER(StepOptions)
        L.adamw_fp8_step.argtypes = [P, P, P, P, P, P, i64, A, P]
        L.adamw_fp8_step_ex.argtypes = [P, P, P, P, P, P, i64, A, O, P]
        L.fold_adamw_fp8_step.argtypes = [P, P, P, P, P, P, P, A, O, P]
        L.fold_adamw_fp8_step_unpack.argtypes = [P, P, P, P, P, P, P, P, P, A, O, P]
        L.fold_adamw_fp8_step_unpack_t.argtypes = [P, P, P, P, P, P, P, P, P, P, P, A, O, P]
        L.unpack_fp8.argtypes = [P, P, P, P, P, P]
        L.bfz_e4m3_encode.argtypes = [P, P, i64, P]
        L.bfz_transpose_pow2.argtypes = [P, P, P, P, P, P]
        L.bfz_last_error.argtypes = []
        L.bfz_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _check(rc):
    if rc != BFZ_OK:
        raise BfzError(rc, lib().bfz_last_error().decode())
    return rc


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev(t, dtype, name, numel=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name}: need a contiguous {dtype} CUDA tensor")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")
    return C.c_void_p(t.data_ptr())


def _tile_array(t, q, name):
    """(pointer, tile stride in floats or None) of a shard array of q FP32
    tiles: a contiguous tensor of at least q * 16384 elements (stride
    16384), or a 2-D view (>= q, 16384) whose rows are the tiles, strides
    (S, 1) -- e.g. state[:, 0] of a (q, 3, 16384) tensor, the interleaved
    layout.  A single-row view has no stride of its own (None)."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32:
        raise TypeError(f"{name}: need a float32 CUDA tensor")
    if t.dim() == 2 and t.shape[1] == TILE_ELEMS and t.stride(1) == 1:
        if t.shape[0] < q:
            raise ValueError(f"{name}: needs at least {q} tiles, has {t.shape[0]}")
        return C.c_void_p(t.data_ptr()), (t.stride(0) if t.shape[0] > 1 else None)
    if t.is_contiguous():
        if t.numel() < q * TILE_ELEMS:
            raise ValueError(f"{name}: needs at least {q * TILE_ELEMS} elements, has {t.numel()}")
        return C.c_void_p(t.data_ptr()), TILE_ELEMS
    raise TypeError(f"{name}: need a contiguous tensor or a (tiles, 16384) view of unit inner stride")


def _hparams(hp):
    return AdamW(**hp) if isinstance(hp, dict) else hp


def _state(master, m, v, q, scale_pow2):
    """Pointers of master, m, v and the step options: scale_pow2 and their
    common tile stride (they must agree; irrelevant when q <= 1)."""
    arrs = [_tile_array(t, q, n) for t, n in ((master, "master"), (m, "m"), (v, "v"))]
    strides = {st for _, st in arrs if st is not None}
    if q <= 1 or not strides:
        stride = TILE_ELEMS
    elif len(strides) == 1:
        stride = strides.pop()
    else:
        raise ValueError(f"master, m and v have different tile strides {sorted(strides)}")
    opts = StepOptions(scale_pow2=int(bool(scale_pow2)), reserved=0,
                       state_stride=0 if stride == TILE_ELEMS else stride)
    return [a for a, _ in arrs], opts


class Plan:
    """Rank `rank`'s block-wise split of the weights `dims` over D ranks.

    dims: sequence of (E, H, W) (E experts of H x W; E = 1 for a matrix).
    The planner runs on the host; bfz_plan_create copies the tile table to
    the current device when a device is visible (on a host without one the
    plan is host-only: table queries work, device calls raise).
    """

    def __init__(self, dims, D=1, rank=0):
        self.dims = [tuple(int(x) for x in d) for d in dims]
        arr = (C.c_int64 * (3 * max(1, len(self.dims))))(*[x for d in self.dims for x in d])
        h = C.c_void_p()
        _check(lib().bfz_plan_create(C.cast(arr, C.c_void_p), len(self.dims), D, rank, C.byref(h)))
        self._h = h
        self.D, self.rank = D, rank

    def upload(self):
        """Copy the table to the current device if the plan has none yet."""
        _check(lib().bfz_plan_upload(self._h))

    @property
    def handle(self):
        return self._h

    @property
    def shard_tiles(self):
        return int(lib().bfz_plan_shard_tiles(self._h))

    @property
    def owned_tiles(self):
        return int(lib().bfz_plan_owned_tiles(self._h))

    @property
    def total_tiles(self):
        return int(lib().bfz_plan_total_tiles(self._h))

    def table(self):
        """numpy int64 [q, 6]: weight, expert, tile row, tile col, valid rows, valid cols."""
        import numpy as np
        out = np.empty((self.shard_tiles, 6), dtype=np.int64)
        _check(lib().bfz_plan_table(self._h, out.ctypes.data_as(C.c_void_p)))
        return out

    def tile(self, slot):
        out = (C.c_int64 * 6)()
        _check(lib().bfz_plan_tile(self._h, slot, C.cast(out, C.c_void_p)))
        return tuple(out)

    def close(self):
        if self._h:
            lib().bfz_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def paramwise_split(dims, D):
    """The page's param-wise split, for comparison: (bucket_of_param int32 [n],
    bucket_elems int64 [D])."""
    import numpy as np
    flat = (C.c_int64 * (3 * max(1, len(dims))))(*[int(x) for d in dims for x in d])
    bop = np.empty(len(dims), dtype=np.int32)
    be = np.empty(D, dtype=np.int64)
    _check(lib().bfz_paramwise_split(C.cast(flat, C.c_void_p), len(dims), D,
                                     bop.ctypes.data_as(C.c_void_p), be.ctypes.data_as(C.c_void_p)))
    return bop, be


def _ptr_array(tensors, dtype, name, sizes):
    """Host array of the per-weight device pointers; tensor p (or None) must
    hold at least sizes[p] elements -- the kernels address it through the
    plan's table, so a smaller tensor would be read or written past its end."""
    n = len(sizes)
    if len(tensors) > n:
        raise ValueError(f"{name}: {len(tensors)} tensors for {n} weights")
    arr = (C.c_void_p * max(1, n))()
    for k in range(n):
        t = tensors[k] if k < len(tensors) else None
        if t is not None:
            arr[k] = _dev(t, dtype, f"{name}[{k}]", sizes[k]).value
    return arr


def _weight_sizes(plan):
    """Elements of each row-major weight (E H W)."""
    return [E * H * W for E, H, W in plan.dims]


def _grid_sizes(plan):
    """Cells of each row-major scale grid (E ceil(H/128) ceil(W/128))."""
    return [E * (-(-H // TILE)) * (-(-W // TILE)) for E, H, W in plan.dims]


def _t_grid_sizes(plan):
    """Cells of each transposed copy's scale grid (E W ceil(H/128))."""
    return [E * W * (-(-H // TILE)) for E, H, W in plan.dims]


def pack_shard(plan: Plan, srcs, dst, stream=None):
    """Fold the weights' row-major FP32 tensors (srcs[p], or None for weights
    the rank does not touch) into the tile-major shard dst: q * 16384
    contiguous floats (pack_shard), or a (>= q, 16384) view whose tiles sit
    S floats apart, e.g. master = state[:, 0] of the interleaved layout
    (pack_shard_strided)."""
    import torch
    arr = _ptr_array(srcs, torch.float32, "srcs", _weight_sizes(plan))
    d, stride = _tile_array(dst, plan.shard_tiles, "dst")
    if stride in (None, TILE_ELEMS):
        _check(lib().pack_shard(plan.handle, C.cast(arr, C.c_void_p), d, _stream(stream)))
    else:
        _check(lib().pack_shard_strided(plan.handle, C.cast(arr, C.c_void_p), d, stride,
                                        _stream(stream)))


def pack_shard_strided(plan: Plan, srcs, dst, dst_stride, stream=None):
    """pack_shard into a flat float32 buffer whose slot s starts at
    s * dst_stride floats (dst must hold (q - 1) * dst_stride + 16384
    floats); pack_shard does the same given a (q, 16384) view."""
    import torch
    q = plan.shard_tiles
    need = (q - 1) * int(dst_stride) + TILE_ELEMS if q else 0
    arr = _ptr_array(srcs, torch.float32, "srcs", _weight_sizes(plan))
    d = _dev(dst, torch.float32, "dst", need)
    _check(lib().pack_shard_strided(plan.handle, C.cast(arr, C.c_void_p), d, int(dst_stride),
                                    _stream(stream)))


def adamw_fp8_step(master, grad, m, v, codes, scale_inv, hp, n_tiles=None, scale_pow2=False,
                   stream=None):
    """Fused AdamW + per-tile E4M3 requant over n_tiles whole tiles (default:
    all of master).  hp: AdamW, or a dict of its fields.  master / m / v:
    contiguous, or (tiles, 16384) views with a common tile stride (the
    interleaved layout: state[:, 0], state[:, 1], state[:, 2] of a
    (q, 3, 16384) tensor).  Plain scales on three tile-major arrays call
    adamw_fp8_step itself; anything else adamw_fp8_step_ex."""
    import torch
    if n_tiles is None:
        if master.dim() == 2 and master.shape[1] == TILE_ELEMS:
            n_tiles = master.shape[0]
        elif master.numel() % TILE_ELEMS:
            raise ValueError("master is not a whole number of tiles")
        else:
            n_tiles = master.numel() // TILE_ELEMS
    n = n_tiles * TILE_ELEMS
    (p, mm, vv), opts = _state(master, m, v, n_tiles, scale_pow2)
    args = [p, _dev(grad, torch.float32, "grad", n), mm, vv,
            _dev(codes, torch.uint8, "codes", n), _dev(scale_inv, torch.float32, "scale_inv", n_tiles)]
    hp = _hparams(hp)
    if opts.scale_pow2 == 0 and opts.state_stride == 0:
        _check(lib().adamw_fp8_step(*args, n_tiles, C.byref(hp), _stream(stream)))
    else:
        _check(lib().adamw_fp8_step_ex(*args, n_tiles, C.byref(hp), C.byref(opts), _stream(stream)))


def fold_adamw_fp8_step(plan: Plan, grads, master, m, v, codes, scale_inv, hp, scale_pow2=False,
                        stream=None):
    """pack_shard of the row-major gradients grads[p] and adamw_fp8_step over
    the whole shard in one pass (the folded gradient is never stored)."""
    import torch
    arr = _ptr_array(grads, torch.float32, "grads", _weight_sizes(plan))
    q = plan.shard_tiles
    n = q * TILE_ELEMS
    (p, mm, vv), opts = _state(master, m, v, q, scale_pow2)
    args = [p, mm, vv, _dev(codes, torch.uint8, "codes", n),
            _dev(scale_inv, torch.float32, "scale_inv", q)]
    _check(lib().fold_adamw_fp8_step(plan.handle, C.cast(arr, C.c_void_p), *args,
                                     C.byref(_hparams(hp)), C.byref(opts), _stream(stream)))


def fold_adamw_fp8_step_unpack(plan: Plan, grads, master, m, v, codes, scale_inv, dst_fp8,
                               dst_scale, hp, scale_pow2=False, stream=None):
    """fold_adamw_fp8_step and unpack_fp8 in one pass.  codes / scale_inv may
    both be None (no tile-major copy of the codes)."""
    import torch
    if (codes is None) != (scale_inv is None):
        raise ValueError("codes and scale_inv: give both or neither")
    q = plan.shard_tiles
    g = _ptr_array(grads, torch.float32, "grads", _weight_sizes(plan))
    a8 = _ptr_array(dst_fp8, torch.uint8, "dst_fp8", _weight_sizes(plan))
    asc = _ptr_array(dst_scale, torch.float32, "dst_scale", _grid_sizes(plan))
    c = None if codes is None else _dev(codes, torch.uint8, "codes", q * TILE_ELEMS)
    sc = None if scale_inv is None else _dev(scale_inv, torch.float32, "scale_inv", q)
    (p, mm, vv), opts = _state(master, m, v, q, scale_pow2)
    _check(lib().fold_adamw_fp8_step_unpack(
        plan.handle, C.cast(g, C.c_void_p), p, mm, vv, c, sc, C.cast(a8, C.c_void_p),
        C.cast(asc, C.c_void_p), C.byref(_hparams(hp)), C.byref(opts), _stream(stream)))


def fold_adamw_fp8_step_unpack_t(plan: Plan, grads, master, m, v, codes, scale_inv, dst_fp8,
                                 dst_scale, dst_t, dst_t_scale, hp, stream=None):
    """fold_adamw_fp8_step_unpack with power-of-two scales plus the transposed
    copy (dst_t[p] uint8 (E, W, H), dst_t_scale[p] float32 (E, W, ceil(H/128)))
    in one pass (power-of-two scales are implied); codes / scale_inv may
    both be None."""
    import torch
    if (codes is None) != (scale_inv is None):
        raise ValueError("codes and scale_inv: give both or neither")
    q = plan.shard_tiles
    g = _ptr_array(grads, torch.float32, "grads", _weight_sizes(plan))
    a8 = _ptr_array(dst_fp8, torch.uint8, "dst_fp8", _weight_sizes(plan))
    asc = _ptr_array(dst_scale, torch.float32, "dst_scale", _grid_sizes(plan))
    t8 = _ptr_array(dst_t, torch.uint8, "dst_t", _weight_sizes(plan))
    tsc = _ptr_array(dst_t_scale, torch.float32, "dst_t_scale", _t_grid_sizes(plan))
    c = None if codes is None else _dev(codes, torch.uint8, "codes", q * TILE_ELEMS)
    sc = None if scale_inv is None else _dev(scale_inv, torch.float32, "scale_inv", q)
    (p, mm, vv), opts = _state(master, m, v, q, True)
    _check(lib().fold_adamw_fp8_step_unpack_t(
        plan.handle, C.cast(g, C.c_void_p), p, mm, vv, c, sc, C.cast(a8, C.c_void_p),
        C.cast(asc, C.c_void_p), C.cast(t8, C.c_void_p), C.cast(tsc, C.c_void_p),
        C.byref(_hparams(hp)), C.byref(opts), _stream(stream)))


def unpack_fp8(plan: Plan, codes, scale_inv, dst_fp8, dst_scale, stream=None):
    """Unfold the shard's codes and scales into row-major uint8 weights
    dst_fp8[p] (E, H, W) and scale grids dst_scale[p] (E, ceil(H/128), ceil(W/128))."""
    import torch
    a8 = _ptr_array(dst_fp8, torch.uint8, "dst_fp8", _weight_sizes(plan))
    asc = _ptr_array(dst_scale, torch.float32, "dst_scale", _grid_sizes(plan))
    q = plan.shard_tiles
    _check(lib().unpack_fp8(plan.handle, _dev(codes, torch.uint8, "codes", q * TILE_ELEMS),
                            _dev(scale_inv, torch.float32, "scale_inv", q),
                            C.cast(a8, C.c_void_p), C.cast(asc, C.c_void_p), _stream(stream)))


def transpose_pow2(plan: Plan, codes, scale_inv, dst_t, dst_t_scale, stream=None):
    """Transposed copy of the shard's power-of-two-quantized tiles by exponent
    edits: dst_t[p] uint8 (E, W, H), dst_t_scale[p] float32 (E, W, ceil(H/128))."""
    import torch
    q = plan.shard_tiles
    a8 = _ptr_array(dst_t, torch.uint8, "dst_t", _weight_sizes(plan))
    asc = _ptr_array(dst_t_scale, torch.float32, "dst_t_scale", _t_grid_sizes(plan))
    _check(lib().bfz_transpose_pow2(plan.handle, _dev(codes, torch.uint8, "codes", q * TILE_ELEMS),
                                    _dev(scale_inv, torch.float32, "scale_inv", q),
                                    C.cast(a8, C.c_void_p), C.cast(asc, C.c_void_p),
                                    _stream(stream)))


def e4m3_encode(x, out, stream=None):
    """out[k] = E4M3 code of x[k] (the step kernel's rounding), device tensors."""
    import torch
    n = x.numel()
    _check(lib().bfz_e4m3_encode(_dev(x, torch.float32, "x"), _dev(out, torch.uint8, "out", n), n,
                                 _stream(stream)))
