"""CPU oracle for the blockwise-FP8 linear layer (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's cpu_baseline leg, never by the product path.  It shares no code
with the HIP library; see oracle.c for the definitions it follows and the
passages of the pages that fix them.

Arrays are numpy: bf16 tensors are passed as their raw uint16 bit patterns,
E4M3 codes as uint8, scales as float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

_CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall"]


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, no fast-math)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # The mutation tests point this at a deliberately broken build of
    # oracle.c, to show that the pins catch the mistake.
    path = os.environ.get("FP8BLK_ORACLE_LIB")
    if path is None:
        if not os.path.exists(_SO):
            build()
        path = _SO
    lib = ctypes.CDLL(path)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_encode_nearest.restype = ctypes.c_uint8
    lib.orc_e4m3_encode_nearest.argtypes = [ctypes.c_double]
    lib.orc_scale_exponent.restype = ctypes.c_int
    lib.orc_scale_exponent.argtypes = [ctypes.c_double]
    lib.orc_bf16_rne.restype = ctypes.c_uint16
    lib.orc_bf16_rne.argtypes = [ctypes.c_float]
    lib.orc_quantize_rowgroup.restype = None
    lib.orc_quantize_rowgroup.argtypes = [u16p, i64, i64, i64, u8p, i64, f32p, ctypes.c_int]
    lib.orc_quantize_colgroup.restype = None
    lib.orc_quantize_colgroup.argtypes = [u16p, i64, i64, i64, u8p, i64, f32p, ctypes.c_int]
    lib.orc_quantize_block.restype = None
    lib.orc_quantize_block.argtypes = [u16p, i64, i64, i64, u8p, u8p, f32p, ctypes.c_int]
    lib.orc_scale_fp32.restype = ctypes.c_float
    lib.orc_scale_fp32.argtypes = [ctypes.c_float]
    for name in ("orc_gemm_fprop", "orc_gemm_dgrad", "orc_gemm_wgrad"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [i64, i64, i64, u8p, f32p, u8p, f32p, i64p, i64, f32p, f64p, f64p]
    lib.orc_e4m3_encode_array.restype = None
    lib.orc_e4m3_encode_array.argtypes = [f64p, i64, u8p]
    lib.orc_e4m3_encode_nearest_array.restype = None
    lib.orc_e4m3_encode_nearest_array.argtypes = [f64p, i64, u8p]
    lib.orc_bf16_rne_array.restype = None
    lib.orc_bf16_rne_array.argtypes = [f32p, i64, u16p]
    lib.orc_rounding_mode_is_nearest.restype = ctypes.c_int
    lib.orc_rounding_mode_is_nearest.argtypes = []
    _lib = lib
    return lib


def _p(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


# ------------------------------------------------------------------ E4M3 --

def e4m3_decode(codes) -> np.ndarray:
    """Decode E4M3 codes (uint8 array) to float64 (NaN for S.1111.111)."""
    lib = _load()
    table = np.array([lib.orc_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(values) -> np.ndarray:
    """Encoder 1 (arithmetic RNE, saturating) over a float64 array."""
    v = _c(np.asarray(values, dtype=np.float64), np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    _load().orc_e4m3_encode_array(_p(v, ctypes.c_double), v.size, _p(out, ctypes.c_uint8))
    return out.reshape(np.shape(values))


def e4m3_encode_nearest(values) -> np.ndarray:
    """Encoder 2 (nearest-code search, ties to even code) over a float64 array."""
    v = _c(np.asarray(values, dtype=np.float64), np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    _load().orc_e4m3_encode_nearest_array(_p(v, ctypes.c_double), v.size, _p(out, ctypes.c_uint8))
    return out.reshape(np.shape(values))


def scale_exponent(amax: float) -> int:
    return int(_load().orc_scale_exponent(float(amax)))


def bf16_rne(values) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even."""
    v = _c(np.asarray(values, dtype=np.float32), np.float32).ravel()
    out = np.empty(v.size, dtype=np.uint16)
    _load().orc_bf16_rne_array(_p(v, ctypes.c_float), v.size, _p(out, ctypes.c_uint16))
    return out.reshape(np.shape(values))


def bf16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rounding_mode_is_nearest() -> bool:
    return bool(_load().orc_rounding_mode_is_nearest())


# ------------------------------------------------------------ quantizers --

SCALE_POW2, SCALE_FP32 = 0, 1   # the scale rules (`mode` of the quantizers)


def scale_fp32(amax: float) -> float:
    """The amax / 448 rule's scale of a group with this (bf16-exact) amax."""
    return float(_load().orc_scale_fp32(float(amax)))


def quantize_rowgroup(x: np.ndarray, cols: int | None = None, mode: int = SCALE_POW2):
    """Row groups of 128 along the last axis.  x: uint16 [rows, ld_x] (bf16 bits);
    the first `cols` columns are quantized.  Returns (q [rows, cols] uint8,
    s [rows, cols/128] float32)."""
    x = _c(x, np.uint16)
    rows, ld = x.shape
    cols = ld if cols is None else cols
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows, cols // 128), dtype=np.float32)
    _load().orc_quantize_rowgroup(_p(x, ctypes.c_uint16), rows, cols, ld,
                                  _p(q, ctypes.c_uint8), cols, _p(s, ctypes.c_float), mode)
    return q, s


def quantize_colgroup(x: np.ndarray, cols: int | None = None, mode: int = SCALE_POW2):
    """Groups of 128 consecutive rows per column, output transposed.
    Returns (qT [cols, rows] uint8, sT [cols, rows/128] float32)."""
    x = _c(x, np.uint16)
    rows, ld = x.shape
    cols = ld if cols is None else cols
    qT = np.empty((cols, rows), dtype=np.uint8)
    sT = np.empty((cols, rows // 128), dtype=np.float32)
    _load().orc_quantize_colgroup(_p(x, ctypes.c_uint16), rows, cols, ld,
                                  _p(qT, ctypes.c_uint8), rows, _p(sT, ctypes.c_float), mode)
    return qT, sT


def quantize_block(w: np.ndarray, transpose: bool = True, mode: int = SCALE_POW2):
    """128x128 blocks.  Returns (q [rows, cols], qT [cols, rows] or None,
    s [rows/128, cols/128])."""
    w = _c(w, np.uint16)
    rows, cols = w.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    qT = np.empty((cols, rows), dtype=np.uint8) if transpose else None
    s = np.empty((rows // 128, cols // 128), dtype=np.float32)
    _load().orc_quantize_block(_p(w, ctypes.c_uint16), rows, cols, cols, _p(q, ctypes.c_uint8),
                               _p(qT, ctypes.c_uint8) if transpose else None,
                               _p(s, ctypes.c_float), mode)
    return q, qT, s


# ------------------------------------------------------------------ GEMMs --

def _gemm(fn, M, N, K, a, sa, b, sb, rows, ncols):
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    nr = rows.size
    y32 = np.empty((nr, ncols), dtype=np.float32)
    y64 = np.empty((nr, ncols), dtype=np.float64)
    bnd = np.empty((nr, ncols), dtype=np.float64)
    fn(M, N, K, _p(a, ctypes.c_uint8), _p(sa, ctypes.c_float), _p(b, ctypes.c_uint8),
       _p(sb, ctypes.c_float), _p(rows, ctypes.c_int64), nr,
       _p(y32, ctypes.c_float), _p(y64, ctypes.c_double), _p(bnd, ctypes.c_double))
    return y32, y64, bnd


def gemm_fprop(qx, sx, qw, sw, rows=None):
    """Y = X W^T on rows `rows` of Y (default: all).  Returns (y32, y64, bound)."""
    M, K = qx.shape
    N = qw.shape[0]
    rows = np.arange(M) if rows is None else rows
    return _gemm(_load().orc_gemm_fprop, M, N, K, qx, sx, qw, sw, rows, N)


def gemm_dgrad(qdy, sdy, qw, sw, rows=None):
    """dX = dY W on rows `rows` of dX, W read as [N][K] directly."""
    M, N = qdy.shape
    K = qw.shape[1]
    rows = np.arange(M) if rows is None else rows
    return _gemm(_load().orc_gemm_dgrad, M, N, K, qdy, sdy, qw, sw, rows, K)


def gemm_wgrad(qdyT, sdyT, qxT, sxT, rows=None):
    """dW = dY^T X on rows `rows` of dW (i.e. output features n)."""
    N, M = qdyT.shape
    K = qxT.shape[0]
    rows = np.arange(N) if rows is None else rows
    return _gemm(_load().orc_gemm_wgrad, M, N, K, qdyT, sdyT, qxT, sxT, rows, K)
