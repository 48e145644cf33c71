"""ctypes front of the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The product library
(blockwise_fp8_zero_amd) never touches it, and it never touches the product.

All arrays are numpy arrays on the host.  Shapes follow oracle.h: a tile is
16384 contiguous float32 values (128 rows of 128), a plan table is q rows of
{param, expert, tile_row, tile_col, valid_rows, valid_cols}.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
TILE = 128
TILE_ELEMS = TILE * TILE

_lib = None


class HParams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("step", C.c_int64)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        L.ora_e4m3_decode.argtypes = [C.c_uint8]
        L.ora_e4m3_decode.restype = C.c_double
        L.ora_e4m3_encode.argtypes = [C.c_float]
        L.ora_e4m3_encode.restype = C.c_uint8
        L.ora_e4m3_near_midpoint.argtypes = [C.c_float, C.c_double]
        L.ora_e4m3_near_midpoint.restype = C.c_int
        L.ora_e4m3_encode_array.argtypes = [P, P, C.c_int64]
        L.ora_total_tiles.argtypes = [P, C.c_int32]
        L.ora_total_tiles.restype = C.c_int64
        L.ora_plan.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, P, P, P]
        L.ora_plan.restype = C.c_int
        L.ora_paramwise_split.argtypes = [P, C.c_int32, C.c_int32, P, P]
        L.ora_paramwise_split.restype = C.c_int
        L.ora_fold_tile.argtypes = [P, C.c_int64, C.c_int64, C.c_int64, C.c_int64, C.c_int64, P]
        L.ora_pack.argtypes = [P, C.c_int32, P, P, C.c_int64, P]
        L.ora_unpack.argtypes = [P, C.c_int32, P, P, P, C.c_int64, P, P]
        L.ora_adamw.argtypes = [P, P, P, P, C.c_int64, C.POINTER(HParams)]
        L.ora_quant_tiles.argtypes = [P, C.c_int64, P, P, P, C.c_double]
        L.ora_step.argtypes = [P, P, P, P, C.c_int64, C.POINTER(HParams), P, P, P, C.c_double]
        L.ora_transpose_pow2.argtypes = [P, C.c_int32, P, P, P, C.c_int64, P, P]
        L.ora_pow2_scale.argtypes = [C.c_float]
        L.ora_pow2_scale.restype = C.c_float
        L.ora_quant_tiles_mode.argtypes = [P, C.c_int64, P, P, P, C.c_double, C.c_int]
        L.ora_step_mode.argtypes = [P, P, P, P, C.c_int64, C.POINTER(HParams), P, P, P, C.c_double,
                                    C.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _need(a, dtype, name):
    if not (isinstance(a, np.ndarray) and a.dtype == dtype and a.flags.c_contiguous):
        raise TypeError(f"{name}: need a C-contiguous {np.dtype(dtype).name} numpy array")
    return a


def hparams(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1):
    return HParams(lr, beta1, beta2, eps, weight_decay, step)


# ---- E4M3 -------------------------------------------------------------
def e4m3_decode(code: int) -> float:
    return lib().ora_e4m3_decode(int(code))


def e4m3_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().ora_e4m3_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def e4m3_near_midpoint(y: float, rel: float = 1e-6) -> bool:
    return bool(lib().ora_e4m3_near_midpoint(float(y), rel))


# ---- plan ---------------------------------------------------------------
def _dims_array(dims):
    d = np.ascontiguousarray(np.asarray(dims, dtype=np.int64).reshape(-1, 3))
    return d


def total_tiles(dims) -> int:
    d = _dims_array(dims)
    return int(lib().ora_total_tiles(_ptr(d), d.shape[0]))


def plan(dims, D: int, rank: int):
    """Returns (q, owned, table[q, 6]) or raises ValueError on bad input."""
    d = _dims_array(dims)
    q = C.c_int64()
    owned = C.c_int64()
    rc = lib().ora_plan(_ptr(d), d.shape[0], D, rank, C.byref(q), C.byref(owned), None)
    if rc != 0:
        raise ValueError("oracle plan: invalid arguments")
    table = np.empty((q.value, 6), dtype=np.int64)
    lib().ora_plan(_ptr(d), d.shape[0], D, rank, C.byref(q), C.byref(owned), _ptr(table))
    return q.value, owned.value, table


def paramwise_split(dims, D: int):
    """Returns (bucket_of_param int32 [n], bucket_elems int64 [D])."""
    d = _dims_array(dims)
    bop = np.empty(d.shape[0], dtype=np.int32)
    be = np.empty(D, dtype=np.int64)
    if lib().ora_paramwise_split(_ptr(d), d.shape[0], D, _ptr(bop), _ptr(be)) != 0:
        raise ValueError("oracle paramwise_split: invalid arguments")
    return bop, be


# ---- fold / unfold --------------------------------------------------------
def fold_tile(src: np.ndarray, e: int, i: int, j: int) -> np.ndarray:
    """src: row-major float32 array of shape (E, H, W)."""
    _need(src, np.float32, "src")
    E, H, W = src.shape
    out = np.empty(TILE_ELEMS, dtype=np.float32)
    lib().ora_fold_tile(_ptr(src), H, W, e, i, j, _ptr(out))
    return out


def pack(dims, srcs, table) -> np.ndarray:
    """srcs: list of row-major float32 arrays (E, H, W) or None per param."""
    d = _dims_array(dims)
    table = _need(np.ascontiguousarray(table, dtype=np.int64), np.int64, "table")
    q = table.shape[0]
    ptrs = (C.c_void_p * max(1, d.shape[0]))()
    for k, s in enumerate(srcs):
        if s is not None:
            _need(s, np.float32, f"srcs[{k}]")
            ptrs[k] = s.ctypes.data
    out = np.empty(q * TILE_ELEMS, dtype=np.float32)
    lib().ora_pack(_ptr(d), d.shape[0], C.cast(ptrs, C.c_void_p), _ptr(table), q, _ptr(out))
    return out


def unpack(dims, codes, scale_inv, table, dst_codes, dst_scale):
    """dst_codes / dst_scale: per-param uint8 (E,H,W) / float32 (E,hb,wb)
    arrays (or None), written in place for the owned slots."""
    d = _dims_array(dims)
    _need(codes, np.uint8, "codes")
    _need(scale_inv, np.float32, "scale_inv")
    table = np.ascontiguousarray(table, dtype=np.int64)
    n = max(1, d.shape[0])
    pc = (C.c_void_p * n)()
    ps = (C.c_void_p * n)()
    for k in range(d.shape[0]):
        if dst_codes[k] is not None:
            pc[k] = _need(dst_codes[k], np.uint8, "dst_codes").ctypes.data
            ps[k] = _need(dst_scale[k], np.float32, "dst_scale").ctypes.data
    lib().ora_unpack(_ptr(d), d.shape[0], _ptr(codes), _ptr(scale_inv), _ptr(table),
                     table.shape[0], C.cast(pc, C.c_void_p), C.cast(ps, C.c_void_p))


def transpose_pow2(dims, codes, scale_inv, table, dst_t, dst_t_scale):
    """dst_t / dst_t_scale: per-param uint8 (E, W, H) / float32 (E, W, ceil(H/128))
    arrays (or None), written for the owned slots."""
    d = _dims_array(dims)
    _need(codes, np.uint8, "codes")
    _need(scale_inv, np.float32, "scale_inv")
    table = np.ascontiguousarray(table, dtype=np.int64)
    n = max(1, d.shape[0])
    pc = (C.c_void_p * n)()
    ps = (C.c_void_p * n)()
    for k in range(d.shape[0]):
        if dst_t[k] is not None:
            pc[k] = _need(dst_t[k], np.uint8, "dst_t").ctypes.data
            ps[k] = _need(dst_t_scale[k], np.float32, "dst_t_scale").ctypes.data
    lib().ora_transpose_pow2(_ptr(d), d.shape[0], _ptr(codes), _ptr(scale_inv), _ptr(table),
                             table.shape[0], C.cast(pc, C.c_void_p), C.cast(ps, C.c_void_p))


# ---- AdamW, quant, step ---------------------------------------------------
def adamw(p, g, m, v, hp: HParams):
    """In place on float32 arrays of equal size."""
    for a, nme in ((p, "p"), (g, "g"), (m, "m"), (v, "v")):
        _need(a, np.float32, nme)
    assert p.size == g.size == m.size == v.size
    lib().ora_adamw(_ptr(p), _ptr(g), _ptr(m), _ptr(v), p.size, C.byref(hp))


def pow2_scale(amax: float) -> float:
    return float(lib().ora_pow2_scale(amax))


def quant_tiles(p, rel: float = 1e-6, pow2: bool = False):
    """Returns (codes uint8 [n], scale_inv float32 [n_tiles], near_mid uint8 [n])."""
    _need(p, np.float32, "p")
    assert p.size % TILE_ELEMS == 0
    nt = p.size // TILE_ELEMS
    codes = np.empty(p.size, dtype=np.uint8)
    scale = np.empty(nt, dtype=np.float32)
    near = np.empty(p.size, dtype=np.uint8)
    lib().ora_quant_tiles_mode(_ptr(p), nt, _ptr(codes), _ptr(scale), _ptr(near), rel, int(pow2))
    return codes, scale, near


def step(p, g, m, v, hp: HParams, rel: float = 1e-6, pow2: bool = False):
    """Fused reference step in place on p, m, v; returns (codes, scale_inv, near_mid)."""
    for a, nme in ((p, "p"), (g, "g"), (m, "m"), (v, "v")):
        _need(a, np.float32, nme)
    assert p.size % TILE_ELEMS == 0 and p.size == g.size == m.size == v.size
    nt = p.size // TILE_ELEMS
    codes = np.empty(p.size, dtype=np.uint8)
    scale = np.empty(nt, dtype=np.float32)
    near = np.empty(p.size, dtype=np.uint8)
    lib().ora_step_mode(_ptr(p), _ptr(g), _ptr(m), _ptr(v), nt, C.byref(hp), _ptr(codes),
                        _ptr(scale), _ptr(near), rel, int(pow2))
    return codes, scale, near
