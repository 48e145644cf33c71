"""Seeded, counter-based synthetic inputs (ctypes front of libsynth.so).

Serves both sides of every parity check: fill_host() regenerates any slice
on the CPU for the oracle, fill_device() fills full-size GPU buffers, and
the two are bit-identical by construction (see synth.hip).  Holds none of
the optimizer's or the quantizer's arithmetic.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynth.so")

NORMAL, T3, T3_SQUARED, EXPERT_LOGU, ZERO = 0, 1, 2, 3, 4


class Recipe(C.Structure):
    _fields_ = [
        ("key", C.c_uint64), ("kind", C.c_int32), ("reserved", C.c_int32),
        ("scale", C.c_double), ("logu_lo", C.c_double), ("logu_hi", C.c_double),
        ("expert_key", C.c_uint64), ("zero_tile_prob", C.c_double), ("zero_key", C.c_uint64),
        ("H", C.c_int64), ("W", C.c_int64),
    ]

    def __repr__(self):
        return (f"Recipe(kind={self.kind}, scale={self.scale}, H={self.H}, W={self.W}, "
                f"zero_tile_prob={self.zero_tile_prob})")


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        u64, i64, d, P = C.c_uint64, C.c_int64, C.c_double, C.c_void_p
        L.synth_key.argtypes = [u64] * 5
        L.synth_key.restype = u64
        for name in ("synth_uniform", "synth_normal", "synth_student_t3"):
            getattr(L, name).argtypes = [u64, u64]
            getattr(L, name).restype = d
        for name in ("synth_ln", "synth_exp", "synth_sqrt", "synth_cos_turns"):
            getattr(L, name).argtypes = [d]
            getattr(L, name).restype = d
        L.synth_fill_host.argtypes = [P, i64, i64, C.POINTER(Recipe)]
        L.synth_fill_rect_host.argtypes = [P, i64, i64, i64, i64, i64, C.POINTER(Recipe)]
        L.synth_fill_device.argtypes = [P, i64, i64, C.POINTER(Recipe), P]
        _lib = L
    return _lib


def key(seed, config, array, param, step=0) -> int:
    return int(lib().synth_key(seed, config, array, param, step))


def recipe(kind, key_, H, W, scale=1.0, logu=(0.0, 0.0), expert_key=0,
           zero_tile_prob=0.0, zero_key=0) -> Recipe:
    return Recipe(key_, kind, 0, scale, logu[0], logu[1], expert_key, zero_tile_prob,
                  zero_key, H, W)


def fill_host(r: Recipe, lo: int, hi: int) -> np.ndarray:
    out = np.empty(hi - lo, dtype=np.float32)
    if lib().synth_fill_host(out.ctypes.data_as(C.c_void_p), lo, hi, C.byref(r)) != 0:
        raise ValueError("synth_fill_host: bad arguments")
    return out


def fill_rect_host(r: Recipe, e: int, r0: int, nr: int, c0: int, nc: int) -> np.ndarray:
    out = np.empty((nr, nc), dtype=np.float32)
    if lib().synth_fill_rect_host(out.ctypes.data_as(C.c_void_p), e, r0, nr, c0, nc,
                                  C.byref(r)) != 0:
        raise ValueError("synth_fill_rect_host: bad arguments")
    return out


def fill_device(r: Recipe, out, lo: int, hi: int, stream=None) -> None:
    """out: a contiguous float32 CUDA tensor with at least hi - lo elements."""
    import torch
    assert out.is_cuda and out.dtype == torch.float32 and out.is_contiguous()
    assert out.numel() >= hi - lo
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = lib().synth_fill_device(C.c_void_p(out.data_ptr()), lo, hi, C.byref(r), C.c_void_p(s))
    if rc != 0:
        raise RuntimeError(f"synth_fill_device failed ({rc})")
