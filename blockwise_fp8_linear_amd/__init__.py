"""blockwise_fp8_linear_amd -- blockwise-FP8 Transformer linear layer for MI355X.

A thin Python binding over libfp8blk.so (the C ABI in include/fp8blk.h).  The
functions carry the C entry points' names; they take torch tensors on the
current HIP device, check dtype / layout / device, pass raw pointers and the
current stream, and raise RuntimeError on a non-zero status.  Every step of
the computation runs in the library's gfx950 kernels; torch provides device
memory and streams only.

There is no fallback: if libfp8blk.so is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8blk.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fp8blk.h")

# enum values of include/fp8blk.h
FP8BLK_SCALE_POW2 = 0
FP8BLK_SCALE_FP32 = 1
FP8BLK_OUT_BF16 = 0
FP8BLK_OUT_FP32 = 1
FP8BLK_OUT_FP32_ACCUM = 2
FP8BLK_OP_FPROP = 0
FP8BLK_OP_DGRAD = 1
FP8BLK_OP_WGRAD = 2
FP8BLK_OP_BACKWARD = 3
FP8BLK_OP_DGRAD_W = 4
FP8BLK_ALGO_DEFAULT = 0
FP8BLK_ALGO_PROMOTE = 1
FP8BLK_ALGO_SCALED_MFMA = 2

_lib = None


class _BlockJob(ctypes.Structure):
    # struct fp8blk_block_job of include/fp8blk.h
    _fields_ = [("w", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld_w", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("qT", ctypes.c_void_p), ("s", ctypes.c_void_p)]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfp8blk.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m blockwise_fp8_linear_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "fp8_quantize_rowgroup": [vp, i64, i64, i64, vp, i64, vp, i32, vp],
        "fp8_quantize_colgroup": [vp, i64, i64, i64, vp, i64, vp, i32, vp],
        "fp8_quantize_block": [vp, i64, i64, i64, vp, vp, vp, i32, vp],
        "fp8_quantize_dual": [vp, i64, i64, i64, vp, i64, vp, vp, i64, vp, i32, vp],
        "fp8_block_gemm_fprop": [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp],
        "fp8_block_gemm_dgrad": [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp],
        "fp8_block_gemm_wgrad": [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, sz, vp],
        "fp8_block_gemm": [i32, i64, i64, i64, vp, vp, vp, vp, vp, i32, i32, vp, sz, vp],
        "fp8_block_gemm_backward": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, vp, sz, vp],
        "fp8_block_gemm_dgrad_w": [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp],
        "fp8_block_gemm_backward_w": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, vp, sz, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.fp8_quantize_block_batch.argtypes = [ctypes.POINTER(_BlockJob), i32, i32, vp]
    lib.fp8_quantize_block_batch.restype = ctypes.c_int
    lib.fp8_block_gemm_workspace_size.argtypes = [i32, i64, i64, i64]
    lib.fp8_block_gemm_workspace_size.restype = ctypes.c_size_t
    lib.fp8_status_string.argtypes = [i32]
    lib.fp8_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/fp8blk.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(fp8_\w+)\s*\(", text, re.M)))


def fp8_status_string(status: int) -> str:
    return load_library().fp8_status_string(int(status)).decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(fp8_status_string(rc))


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _dev(t, dtype, name, ndim=2):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: on {t.device}, but the library launches on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {t.dim()}")
    if ndim == 2 and t.stride(1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return t


def _dense(t, dtype, name):
    _dev(t, dtype, name)
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


# -------------------------------------------------------------- quantizers --

def fp8_quantize_rowgroup(x, q=None, s=None, stream=None, scale_mode=FP8BLK_SCALE_POW2):
    """Groups of 128 along the last dim.  x: bf16 [rows, cols] (row stride may
    exceed cols).  Returns (q uint8 [rows, cols], s fp32 [rows, cols/128]).
    scale_mode (every quantizer): FP8BLK_SCALE_POW2 (power-of-two scales) or
    FP8BLK_SCALE_FP32 (amax / 448; GEMMs then need FP8BLK_ALGO_PROMOTE)."""
    import torch
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else _dev(q, torch.uint8, "q")
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device) if s is None else _dense(s, torch.float32, "s")
    _check(load_library().fp8_quantize_rowgroup(x.data_ptr(), rows, cols, x.stride(0), q.data_ptr(), q.stride(0),
                                                s.data_ptr(), scale_mode, _stream(stream)))
    return q, s


def fp8_quantize_colgroup(x, qT=None, sT=None, stream=None, scale_mode=FP8BLK_SCALE_POW2):
    """Groups of 128 consecutive rows per column, written transposed.
    Returns (qT uint8 [cols, rows], sT fp32 [cols, rows/128])."""
    import torch
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if qT is None else _dev(qT, torch.uint8, "qT")
    sT = (torch.empty((cols, rows // 128), dtype=torch.float32, device=x.device) if sT is None
          else _dense(sT, torch.float32, "sT"))
    _check(load_library().fp8_quantize_colgroup(x.data_ptr(), rows, cols, x.stride(0), qT.data_ptr(), qT.stride(0),
                                                sT.data_ptr(), scale_mode, _stream(stream)))
    return qT, sT


def fp8_quantize_dual(x, q=None, s=None, qT=None, sT=None, stream=None, scale_mode=FP8BLK_SCALE_POW2):
    """Row groups and column groups in one pass.  Returns (q, s, qT, sT) equal
    to fp8_quantize_rowgroup(x) + fp8_quantize_colgroup(x)."""
    import torch
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else _dev(q, torch.uint8, "q")
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device) if s is None else _dense(s, torch.float32, "s")
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if qT is None else _dev(qT, torch.uint8, "qT")
    sT = (torch.empty((cols, rows // 128), dtype=torch.float32, device=x.device) if sT is None
          else _dense(sT, torch.float32, "sT"))
    _check(load_library().fp8_quantize_dual(x.data_ptr(), rows, cols, x.stride(0), q.data_ptr(), q.stride(0),
                                            s.data_ptr(), qT.data_ptr(), qT.stride(0), sT.data_ptr(),
                                            scale_mode, _stream(stream)))
    return q, s, qT, sT


def fp8_quantize_block_batch(weights, transpose=True, outs=None, stream=None, scale_mode=FP8BLK_SCALE_POW2):
    """Several weights (bf16 [rows, cols] tensors, at most 8) quantized in one
    launch, each as by fp8_quantize_block.  Returns a list of (q, qT or None,
    s); `outs`, if given, is such a list of preallocated outputs."""
    import torch
    n = len(weights)
    jobs = (_BlockJob * n)()
    res = []
    for k, w in enumerate(weights):
        _dev(w, torch.bfloat16, f"weights[{k}]")
        rows, cols = w.shape
        if outs is not None:
            q, qT, s = outs[k]
            _dense(q, torch.uint8, "q")
            _dense(s, torch.float32, "s")
            if qT is not None:
                _dense(qT, torch.uint8, "qT")
        else:
            q = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
            qT = torch.empty((cols, rows), dtype=torch.uint8, device=w.device) if transpose else None
            s = torch.empty((rows // 128, cols // 128), dtype=torch.float32, device=w.device)
        jobs[k] = _BlockJob(w.data_ptr(), rows, cols, w.stride(0), q.data_ptr(),
                            qT.data_ptr() if qT is not None else None, s.data_ptr())
        res.append((q, qT, s))
    _check(load_library().fp8_quantize_block_batch(jobs, n, scale_mode, _stream(stream)))
    return res


def fp8_quantize_block(w, transpose=True, q=None, qT=None, s=None, stream=None, scale_mode=FP8BLK_SCALE_POW2):
    """128x128 blocks.  Returns (q uint8 [rows, cols], qT uint8 [cols, rows] or
    None, s fp32 [rows/128, cols/128])."""
    import torch
    _dev(w, torch.bfloat16, "w")
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=w.device) if q is None else _dense(q, torch.uint8, "q")
    if transpose:
        qT = (torch.empty((cols, rows), dtype=torch.uint8, device=w.device) if qT is None
              else _dense(qT, torch.uint8, "qT"))
    else:
        qT = None
    s = (torch.empty((rows // 128, cols // 128), dtype=torch.float32, device=w.device) if s is None
         else _dense(s, torch.float32, "s"))
    _check(load_library().fp8_quantize_block(w.data_ptr(), rows, cols, w.stride(0), q.data_ptr(),
                                             qT.data_ptr() if qT is not None else None, s.data_ptr(),
                                             scale_mode, _stream(stream)))
    return q, qT, s


# ------------------------------------------------------------------- GEMMs --

def _out(shape, out_dtype, device, out):
    import torch
    if out is not None:
        return _dense(out, out_dtype, "out")
    return torch.empty(shape, dtype=out_dtype, device=device)


def _odt(out_dtype, accumulate=False, out=None):
    import torch
    if accumulate:
        if out_dtype != torch.float32 or out is None:
            raise ValueError("accumulate=True needs out_dtype=torch.float32 and an existing `out` to add to")
        return FP8BLK_OUT_FP32_ACCUM
    if out_dtype == torch.bfloat16:
        return FP8BLK_OUT_BF16
    if out_dtype == torch.float32:
        return FP8BLK_OUT_FP32
    raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")


def fp8_block_gemm_workspace_size(op: int, M: int, N: int, K: int) -> int:
    return int(load_library().fp8_block_gemm_workspace_size(op, M, N, K))


def fp8_block_gemm(op, a, sa, b, sb, M, N, K, out_dtype=None, algo=FP8BLK_ALGO_DEFAULT, out=None,
                   workspace=None, stream=None, accumulate=False):
    """Any of the three contractions with an explicit algorithm (see
    fp8_block_gemm in include/fp8blk.h for the operand roles).  accumulate:
    out += result in fp32 (out_dtype float32, `out` given)."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    for t, n in ((a, "a"), (b, "b")):
        _dense(t, torch.uint8, n)
    for t, n in ((sa, "sa"), (sb, "sb")):
        _dense(t, torch.float32, n)
    shape = {FP8BLK_OP_FPROP: (M, N), FP8BLK_OP_DGRAD: (M, K), FP8BLK_OP_WGRAD: (N, K), FP8BLK_OP_DGRAD_W: (M, K)}[op]
    y = _out(shape, out_dtype, a.device, out)
    need = fp8_block_gemm_workspace_size(op, M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().fp8_block_gemm(op, M, N, K, a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                                         y.data_ptr(), _odt(out_dtype, accumulate, out), algo, wptr, wbytes, _stream(stream)))
    return y


def fp8_block_gemm_fprop(qx, sx, qw, sw, out_dtype=None, out=None, stream=None, accumulate=False):
    """Y = X W^T.  qx [M,K], sx [M,K/128], qw [N,K], sw [N/128,K/128] -> Y [M,N]."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    M, K = qx.shape
    N = qw.shape[0]
    for t, n in ((qx, "qx"), (qw, "qw")):
        _dense(t, torch.uint8, n)
    for t, n in ((sx, "sx"), (sw, "sw")):
        _dense(t, torch.float32, n)
    y = _out((M, N), out_dtype, qx.device, out)
    _check(load_library().fp8_block_gemm_fprop(M, N, K, qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(),
                                               y.data_ptr(), _odt(out_dtype, accumulate, out), _stream(stream)))
    return y


def fp8_block_gemm_dgrad(qdy, sdy, qwT, sw, out_dtype=None, out=None, stream=None, accumulate=False):
    """dX = dY W.  qdy [M,N], sdy [M,N/128], qwT [K,N], sw [N/128,K/128] -> dX [M,K]."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    M, N = qdy.shape
    K = qwT.shape[0]
    for t, n in ((qdy, "qdy"), (qwT, "qwT")):
        _dense(t, torch.uint8, n)
    for t, n in ((sdy, "sdy"), (sw, "sw")):
        _dense(t, torch.float32, n)
    y = _out((M, K), out_dtype, qdy.device, out)
    _check(load_library().fp8_block_gemm_dgrad(M, N, K, qdy.data_ptr(), sdy.data_ptr(), qwT.data_ptr(),
                                               sw.data_ptr(), y.data_ptr(), _odt(out_dtype, accumulate, out), _stream(stream)))
    return y


def fp8_block_gemm_dgrad_w(qdy, sdy, qw, sw, out_dtype=None, out=None, stream=None, accumulate=False):
    """dX = dY W from the weight codes as quantized.  qdy [M,N], sdy [M,N/128],
    qw [N,K], sw [N/128,K/128] -> dX [M,K]."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    M, N = qdy.shape
    K = qw.shape[1]
    for t, n in ((qdy, "qdy"), (qw, "qw")):
        _dense(t, torch.uint8, n)
    for t, n in ((sdy, "sdy"), (sw, "sw")):
        _dense(t, torch.float32, n)
    y = _out((M, K), out_dtype, qdy.device, out)
    _check(load_library().fp8_block_gemm_dgrad_w(M, N, K, qdy.data_ptr(), sdy.data_ptr(), qw.data_ptr(),
                                                 sw.data_ptr(), y.data_ptr(), _odt(out_dtype, accumulate, out),
                                                 _stream(stream)))
    return y


def fp8_block_gemm_wgrad(qdyT, sdyT, qxT, sxT, out_dtype=None, out=None, workspace=None, stream=None,
                         accumulate=False):
    """dW = dY^T X.  qdyT [N,M], sdyT [N,M/128], qxT [K,M], sxT [K,M/128] -> dW [N,K]."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    N, M = qdyT.shape
    K = qxT.shape[0]
    for t, n in ((qdyT, "qdyT"), (qxT, "qxT")):
        _dense(t, torch.uint8, n)
    for t, n in ((sdyT, "sdyT"), (sxT, "sxT")):
        _dense(t, torch.float32, n)
    y = _out((N, K), out_dtype, qdyT.device, out)
    need = fp8_block_gemm_workspace_size(FP8BLK_OP_WGRAD, M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=qdyT.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().fp8_block_gemm_wgrad(M, N, K, qdyT.data_ptr(), sdyT.data_ptr(), qxT.data_ptr(),
                                               sxT.data_ptr(), y.data_ptr(), _odt(out_dtype, accumulate, out), wptr, wbytes,
                                               _stream(stream)))
    return y


def fp8_block_gemm_backward(qdy, sdy, qwT, sw, qdyT, sdyT, qxT, sxT, dx_dtype=None, dw_dtype=None, dx=None,
                            dw=None, workspace=None, stream=None, accumulate_dw=False):
    """Dgrad and Wgrad of one linear in one call.  Operands as for
    fp8_block_gemm_dgrad and fp8_block_gemm_wgrad; returns (dx [M,K], dw [N,K]).
    accumulate_dw: dw += dY^T X in fp32 (dw_dtype float32, `dw` given)."""
    return _backward("fp8_block_gemm_backward", qdy, sdy, qwT, qwT.shape[0], sw, qdyT, sdyT, qxT, sxT, dx_dtype,
                     dw_dtype, dx, dw, workspace, stream, accumulate_dw)


def fp8_block_gemm_backward_w(qdy, sdy, qw, sw, qdyT, sdyT, qxT, sxT, dx_dtype=None, dw_dtype=None, dx=None,
                              dw=None, workspace=None, stream=None, accumulate_dw=False):
    """fp8_block_gemm_backward with Dgrad reading the weight codes qw [N,K] as
    quantized (no transposed copy)."""
    return _backward("fp8_block_gemm_backward_w", qdy, sdy, qw, qw.shape[1], sw, qdyT, sdyT, qxT, sxT, dx_dtype,
                     dw_dtype, dx, dw, workspace, stream, accumulate_dw)


def _backward(fn, qdy, sdy, qwT, K, sw, qdyT, sdyT, qxT, sxT, dx_dtype, dw_dtype, dx, dw, workspace, stream,
              accumulate_dw):
    import torch
    dx_dtype = torch.bfloat16 if dx_dtype is None else dx_dtype
    dw_dtype = torch.bfloat16 if dw_dtype is None else dw_dtype
    M, N = qdy.shape
    for t, n in ((qdy, "qdy"), (qwT, "weight codes"), (qdyT, "qdyT"), (qxT, "qxT")):
        _dense(t, torch.uint8, n)
    for t, n in ((sdy, "sdy"), (sw, "sw"), (sdyT, "sdyT"), (sxT, "sxT")):
        _dense(t, torch.float32, n)
    x = _out((M, K), dx_dtype, qdy.device, dx)
    w = _out((N, K), dw_dtype, qdy.device, dw)
    need = fp8_block_gemm_workspace_size(FP8BLK_OP_BACKWARD, M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=qdy.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(getattr(load_library(), fn)(M, N, K, qdy.data_ptr(), sdy.data_ptr(), qwT.data_ptr(),
                                       sw.data_ptr(), qdyT.data_ptr(), sdyT.data_ptr(), qxT.data_ptr(),
                                       sxT.data_ptr(), x.data_ptr(), _odt(dx_dtype),
                                       w.data_ptr(), _odt(dw_dtype, accumulate_dw, dw), wptr, wbytes,
                                       _stream(stream)))
    return x, w

