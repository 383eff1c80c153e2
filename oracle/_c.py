"""ctypes access to the C oracle (oracle.c).  Test infrastructure only.

Arrays are numpy; bf16 values travel as their uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class AdamHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64),
                ("decoupled", ctypes.c_int32), ("_pad", ctypes.c_int32)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build
            build.build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.orc_bf16_to_f32.argtypes = [P, P, I64]
        L.orc_f32_to_bf16.argtypes = [P, P, I64]
        L.orc_average_bf16.argtypes = [ctypes.c_int32, P, I64, P]
        L.orc_average_f32.argtypes = [ctypes.c_int32, P, I64, P]
        L.orc_accumulate_bf16.argtypes = [P, P, I64]
        L.orc_sumsq_f32.argtypes = [P, I64]
        L.orc_sumsq_f32.restype = ctypes.c_double
        L.orc_clip_coef.argtypes = [ctypes.c_double, ctypes.c_float]
        L.orc_clip_coef.restype = ctypes.c_float
        L.orc_scale_f32.argtypes = [P, I64, ctypes.c_float]
        L.orc_adam_f32.argtypes = [ctypes.POINTER(AdamHParams), I64, P, P, P, P]
        L.orc_adam_f64.argtypes = [ctypes.POINTER(AdamHParams), I64, P, P, P, P]
        L.orc_rank_step_bf16.argtypes = [ctypes.POINTER(AdamHParams), ctypes.c_int32,
                                         P, I64, ctypes.c_float, P, P, P, P, P]
        L.orc_rank_step_f32.argtypes = [ctypes.POINTER(AdamHParams), ctypes.c_int32,
                                        P, I64, ctypes.c_float, P, P, P, P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _ptr_array(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return arr


def hparams(lr, beta1, beta2, eps, weight_decay, step, decoupled):
    return AdamHParams(lr, beta1, beta2, eps, weight_decay, int(step), int(bool(decoupled)), 0)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().orc_bf16_to_f32(_ptr(bits), _ptr(out), bits.size)
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16(_ptr(x), _ptr(out), x.size)
    return out


def average(ranks) -> np.ndarray:
    """Mean over the N rank arrays (all bf16-bits uint16 or all float32)."""
    ranks = [np.ascontiguousarray(r) for r in ranks]
    n = ranks[0].size
    assert all(r.size == n and r.dtype == ranks[0].dtype for r in ranks)
    out = np.empty(n, np.float32)
    if ranks[0].dtype == np.uint16:
        lib().orc_average_bf16(len(ranks), _ptr_array(ranks), n, _ptr(out))
    elif ranks[0].dtype == np.float32:
        lib().orc_average_f32(len(ranks), _ptr_array(ranks), n, _ptr(out))
    else:
        raise TypeError(ranks[0].dtype)
    return out


def accumulate_bf16(acc: np.ndarray, micro: np.ndarray) -> None:
    assert acc.dtype == np.float32 and micro.dtype == np.uint16 and acc.size == micro.size
    lib().orc_accumulate_bf16(_ptr(acc), _ptr(micro), acc.size)


def sumsq(g: np.ndarray) -> float:
    g = np.ascontiguousarray(g, dtype=np.float32)
    return lib().orc_sumsq_f32(_ptr(g), g.size)


def clip_coef(total_sumsq: float, max_norm: float) -> float:
    return lib().orc_clip_coef(total_sumsq, max_norm)


def scale(g: np.ndarray, c: float) -> None:
    assert g.dtype == np.float32
    lib().orc_scale_f32(_ptr(g), g.size, c)


def adam(hp: AdamHParams, g, p, m, v) -> None:
    """In-place fp32 Adam/AdamW step on (p, m, v) with gradient g."""
    for a in (g, p, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    assert g.size == p.size == m.size == v.size
    lib().orc_adam_f32(ctypes.byref(hp), p.size, _ptr(g), _ptr(p), _ptr(m), _ptr(v))


def adam_f64(hp: AdamHParams, g, p, m, v) -> None:
    for a in (g, p, m, v):
        assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    lib().orc_adam_f64(ctypes.byref(hp), p.size, _ptr(g), _ptr(p), _ptr(m), _ptr(v))


def rank_step(hp: AdamHParams, ranks, clip_c, p, m, v, param_out, tmp=None) -> None:
    """average -> clip scale -> Adam -> bf16, over one contiguous run."""
    n = p.size
    tmp = np.empty(n, np.float32) if tmp is None else tmp
    ranks = [np.ascontiguousarray(r) for r in ranks]
    if ranks[0].dtype == np.uint16:
        fn = lib().orc_rank_step_bf16
    else:
        fn = lib().orc_rank_step_f32
    fn(ctypes.byref(hp), len(ranks), _ptr_array(ranks), n, clip_c,
       _ptr(tmp), _ptr(p), _ptr(m), _ptr(v), _ptr(param_out))
