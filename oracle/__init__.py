"""CPU oracle for the fused 3x3 conv + epilogue ops -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and shares no code with it.

Thin ctypes wrapper over ``libx3oracle.so`` (plain C + OpenMP, double
precision; see ``x3_oracle.c`` for the definitions and their sources).
Inputs are numpy float32 arrays (made contiguous here); every result is a
float64 numpy array.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libx3oracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_int = ctypes.c_int
_dbl = ctypes.c_double
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # noqa: PLC0415
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "x3o_conv3x3_bias": [_f32p, _f32p, _f32p, _f64p, _int, _int, _int, _int, _int],
        "x3o_min_tanh2": [_f32p, _f32p, _f32p, _f64p, _int, _int, _int, _int, _int],
        "x3o_min_tanh2_at": [_f32p, _f32p, _f32p, _int, _int, _int, _int, _i64p, _i64, _f64p],
        "x3o_mul_lrelu_gelu": [_f32p, _f32p, _f32p, _f32p, _dbl, _f64p, _int, _int, _int, _int, _int],
        "x3o_mul_lrelu_gelu_tanh": [_f32p, _f32p, _f32p, _f32p, _dbl, _f64p, _int, _int, _int,
                                    _int, _int],
        "x3o_mul_lrelu_gelu_at": [_f32p, _f32p, _f32p, _f32p, _dbl, _int, _int, _int, _i64p, _i64, _f64p],
        "x3o_scale_min": [_f32p, _f32p, _f32p, _dbl, _f64p, _int, _int, _int, _int, _int],
        "x3o_scale_min_at": [_f32p, _f32p, _f32p, _dbl, _int, _int, _int, _int, _i64p, _i64, _f64p],
        "x3o_group_norm": [_f64p, _f32p, _f32p, _int, _dbl, _f64p, _int, _int, _int, _int],
        "x3o_gn_scale_pool_clamp": [_f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _int, _dbl, _int,
                                    _dbl, _dbl, _f64p, _int, _int, _int, _int, _int],
        "x3o_num_threads": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _int if name in ("x3o_gn_scale_pool_clamp", "x3o_num_threads") else None
    _lib = lib
    return lib


def _f32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return a, a.ctypes.data_as(_f32p)


def _shape(x, w):
    B, Cin, H, W = x.shape
    Cout, Cin_w, kh, kw = w.shape
    if Cin_w != Cin or kh != 3 or kw != 3:
        raise ValueError("weight must be [Cout, Cin, 3, 3]")
    return B, Cin, H, W, Cout


def num_threads() -> int:
    return int(_load().x3o_num_threads())


def conv3x3_bias(x, w, b) -> np.ndarray:
    """y = valid 3x3 conv (stride 1) + bias, [B, Cout, H-2, W-2], float64."""
    lib = _load()
    x, xp = _f32(x); w, wp = _f32(w); b, bp = _f32(b)
    B, Cin, H, W, Cout = _shape(x, w)
    y = np.empty((B, Cout, H - 2, W - 2), dtype=np.float64)
    lib.x3o_conv3x3_bias(xp, wp, bp, y.ctypes.data_as(_f64p), B, Cin, H, W, Cout)
    return y


def min_tanh2(x, w, b) -> np.ndarray:
    """tanh(tanh(min over channels of conv)), [B, 1, H-2, W-2]."""
    lib = _load()
    x, xp = _f32(x); w, wp = _f32(w); b, bp = _f32(b)
    B, Cin, H, W, Cout = _shape(x, w)
    out = np.empty((B, 1, H - 2, W - 2), dtype=np.float64)
    lib.x3o_min_tanh2(xp, wp, bp, out.ctypes.data_as(_f64p), B, Cin, H, W, Cout)
    return out


def min_tanh2_at(x, w, b, pix) -> np.ndarray:
    """Sampled epilogue (a): pix is an int64 array of (n, h, w) rows."""
    lib = _load()
    x, xp = _f32(x); w, wp = _f32(w); b, bp = _f32(b)
    B, Cin, H, W, Cout = _shape(x, w)
    pix = np.ascontiguousarray(pix, dtype=np.int64).reshape(-1, 3)
    out = np.empty(pix.shape[0], dtype=np.float64)
    lib.x3o_min_tanh2_at(xp, wp, bp, Cin, H, W, Cout, pix.ctypes.data_as(_i64p),
                         pix.shape[0], out.ctypes.data_as(_f64p))
    return out


def mul_lrelu_gelu(x, w, b, mult, slope=0.01) -> np.ndarray:
    """gelu_erf(leaky_relu(conv * mult[c], slope)), [B, Cout, H-2, W-2]."""
    lib = _load()
    x, xp = _f32(x); w, wp = _f32(w); b, bp = _f32(b); m, mp = _f32(mult)
    B, Cin, H, W, Cout = _shape(x, w)
    out = np.empty((B, Cout, H - 2, W - 2), dtype=np.float64)
    lib.x3o_mul_lrelu_gelu(xp, wp, bp, mp, float(slope), out.ctypes.data_as(_f64p),
                           B, Cin, H, W, Cout)
    return out


def mul_lrelu_gelu_tanh(x, w, b, mult, slope=0.01) -> np.ndarray:
    """gelu_tanh(leaky_relu(conv * mult[c], slope)), [B, Cout, H-2, W-2]."""
    lib = _load()
    x, xp = _f32(x); w, wp = _f32(w); b, bp = _f32(b); m, mp = _f32(mult)
    B, Cin, H, W, Cout = _shape(x, w)
    out = np.empty((B, Cout, H - 2, W - 2), dtype=np.float64)
    lib.x3o_mul_lrelu_gelu_tanh(xp, wp, bp, mp, float(slope), out.ctypes.data_as(_f64p),
                                B, Cin, H, W, Cout)
    return out


def mul_lrelu_gelu_at(x, w, b, mult, el, slope=0.01) -> np.ndarray:
    """Sampled epilogue (b): el is an int64 array of (n, co, h, w) rows."""
    lib = _load()
    x, xp = _f32(x); w, wp = _f32(w); b, bp = _f32(b); m, mp = _f32(mult)
    B, Cin, H, W, Cout = _shape(x, w)
    el = np.ascontiguousarray(el, dtype=np.int64).reshape(-1, 4)
    out = np.empty(el.shape[0], dtype=np.float64)
    lib.x3o_mul_lrelu_gelu_at(xp, wp, bp, mp, float(slope), Cin, H, W,
                              el.ctypes.data_as(_i64p), el.shape[0],
                              out.ctypes.data_as(_f64p))
    return out


def scale_min(x, w, b, scale=2.0) -> np.ndarray:
    """min over channels of (scale * conv), [B, 1, H-2, W-2]."""
    lib = _load()
    x, xp = _f32(x); w, wp = _f32(w); b, bp = _f32(b)
    B, Cin, H, W, Cout = _shape(x, w)
    out = np.empty((B, 1, H - 2, W - 2), dtype=np.float64)
    lib.x3o_scale_min(xp, wp, bp, float(scale), out.ctypes.data_as(_f64p), B, Cin, H, W, Cout)
    return out


def scale_min_at(x, w, b, pix, scale=2.0) -> np.ndarray:
    """Sampled epilogue (c): pix is an int64 array of (n, h, w) rows."""
    lib = _load()
    x, xp = _f32(x); w, wp = _f32(w); b, bp = _f32(b)
    B, Cin, H, W, Cout = _shape(x, w)
    pix = np.ascontiguousarray(pix, dtype=np.int64).reshape(-1, 3)
    out = np.empty(pix.shape[0], dtype=np.float64)
    lib.x3o_scale_min_at(xp, wp, bp, float(scale), Cin, H, W, Cout,
                         pix.ctypes.data_as(_i64p), pix.shape[0], out.ctypes.data_as(_f64p))
    return out


def group_norm(y, groups, eps=1e-5, gamma=None, beta=None) -> np.ndarray:
    """GroupNorm of a float64 [B, C, H, W] array (affine optional)."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float64)
    B, C, HH, WW = y.shape
    if C % groups:
        raise ValueError("C must be divisible by groups")
    gp = bp = None
    if gamma is not None:
        g, gp = _f32(gamma)
    if beta is not None:
        bb, bp = _f32(beta)
    z = np.empty_like(y)
    lib.x3o_group_norm(y.ctypes.data_as(_f64p), gp, bp, groups, float(eps),
                       z.ctypes.data_as(_f64p), B, C, HH, WW)
    return z


def gn_scale_pool_clamp(x, w, b, gamma, beta, scale, groups=16, eps=1e-5,
                        pool_k=4, lo=0.0, hi=1.0) -> np.ndarray:
    """clamp(maxpool_k(GroupNorm(conv) * scale[c]), lo, hi), [B, Cout, P, P]."""
    lib = _load()
    x, xp = _f32(x); w, wp = _f32(w); b, bp = _f32(b)
    g, gp = _f32(gamma); be, bep = _f32(beta); s, sp = _f32(scale)
    B, Cin, H, W, Cout = _shape(x, w)
    Ho, Wo = H - 2, W - 2
    if Ho < pool_k or Wo < pool_k:
        raise ValueError("pool window larger than the conv output")
    Ph, Pw = (Ho - pool_k) // pool_k + 1, (Wo - pool_k) // pool_k + 1
    out = np.empty((B, Cout, Ph, Pw), dtype=np.float64)
    rc = lib.x3o_gn_scale_pool_clamp(xp, wp, bp, gp, bep, sp, groups, float(eps), pool_k,
                                     float(lo), float(hi), out.ctypes.data_as(_f64p),
                                     B, Cin, H, W, Cout)
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out
