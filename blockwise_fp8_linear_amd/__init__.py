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
FP8BLK_ERR_SCRATCH = -8
FP8BLK_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

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
    # torch ships its own HIP runtime under the same soname as the system's.
    # Loaded first, this library would pull in the system copy and torch its
    # own: two runtimes in one process, whose streams and kernels do not mix
    # (every launch fails).  Importing torch first makes the library bind to
    # torch's runtime.
    import torch  # noqa: F401
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
        "fp8_block_gemm": [i32, i64, i64, i64, vp, vp, vp, vp, vp, i32, i32, i32, vp, sz, vp],
        "fp8_block_gemm_backward": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, sz,
                                    vp],
        "fp8_block_gemm_dgrad_w": [i64, i64, i64, vp, vp, vp, vp, vp, i32, vp],
        "fp8_block_gemm_backward_w": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, sz,
                                      vp],
        "fp8_block_gemm_backward_w_noalloc": [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                              vp],
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


def _shape(t, shape, name):
    """The kernels read and write exactly the extents the C call is given, so
    every tensor must have the shape those extents imply: a smaller one would
    be accessed out of bounds on the device."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _on(stream):
    """Context in which tensors the call allocates belong to the stream it
    launches on, so that torch's caching allocator never hands their memory
    to other work before that stream has finished with it."""
    import contextlib
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _new(shape, dtype, device, stream):
    import torch
    with _on(stream):
        return torch.empty(shape, dtype=dtype, device=device)


# -------------------------------------------------------------- quantizers --

def fp8_quantize_rowgroup(x, q=None, s=None, stream=None, scale_mode=FP8BLK_SCALE_POW2):
    """Groups of 128 along the last dim.  x: bf16 [rows, cols] (row stride may
    exceed cols).  Returns (q uint8 [rows, cols], s fp32 [rows, cols/128]).
    scale_mode (every quantizer): FP8BLK_SCALE_POW2 (power-of-two scales) or
    FP8BLK_SCALE_FP32 (amax / 448; GEMMs then need FP8BLK_ALGO_PROMOTE)."""
    import torch
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    q = _new((rows, cols), torch.uint8, x.device, stream) if q is None else _dev(q, torch.uint8, "q")
    s = _new((rows, cols // 128), torch.float32, x.device, stream) if s is None else _dense(s, torch.float32, "s")
    _shape(q, (rows, cols), "q")
    _shape(s, (rows, cols // 128), "s")
    _check(load_library().fp8_quantize_rowgroup(x.data_ptr(), rows, cols, x.stride(0), q.data_ptr(), q.stride(0),
                                                s.data_ptr(), scale_mode, _stream(stream)))
    return q, s


def fp8_quantize_colgroup(x, qT=None, sT=None, stream=None, scale_mode=FP8BLK_SCALE_POW2):
    """Groups of 128 consecutive rows per column, written transposed.
    Returns (qT uint8 [cols, rows], sT fp32 [cols, rows/128])."""
    import torch
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    qT = _new((cols, rows), torch.uint8, x.device, stream) if qT is None else _dev(qT, torch.uint8, "qT")
    sT = _new((cols, rows // 128), torch.float32, x.device, stream) if sT is None else _dense(sT, torch.float32, "sT")
    _shape(qT, (cols, rows), "qT")
    _shape(sT, (cols, rows // 128), "sT")
    _check(load_library().fp8_quantize_colgroup(x.data_ptr(), rows, cols, x.stride(0), qT.data_ptr(), qT.stride(0),
                                                sT.data_ptr(), scale_mode, _stream(stream)))
    return qT, sT


def fp8_quantize_dual(x, q=None, s=None, qT=None, sT=None, stream=None, scale_mode=FP8BLK_SCALE_POW2):
    """Row groups and column groups in one pass.  Returns (q, s, qT, sT) equal
    to fp8_quantize_rowgroup(x) + fp8_quantize_colgroup(x)."""
    import torch
    _dev(x, torch.bfloat16, "x")
    rows, cols = x.shape
    q = _new((rows, cols), torch.uint8, x.device, stream) if q is None else _dev(q, torch.uint8, "q")
    s = _new((rows, cols // 128), torch.float32, x.device, stream) if s is None else _dense(s, torch.float32, "s")
    qT = _new((cols, rows), torch.uint8, x.device, stream) if qT is None else _dev(qT, torch.uint8, "qT")
    sT = _new((cols, rows // 128), torch.float32, x.device, stream) if sT is None else _dense(sT, torch.float32, "sT")
    _shape(q, (rows, cols), "q")
    _shape(s, (rows, cols // 128), "s")
    _shape(qT, (cols, rows), "qT")
    _shape(sT, (cols, rows // 128), "sT")
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
            _shape(_dense(q, torch.uint8, f"outs[{k}] q"), (rows, cols), f"outs[{k}] q")
            _shape(_dense(s, torch.float32, f"outs[{k}] s"), (rows // 128, cols // 128), f"outs[{k}] s")
            if qT is not None:
                _shape(_dense(qT, torch.uint8, f"outs[{k}] qT"), (cols, rows), f"outs[{k}] qT")
        else:
            q = _new((rows, cols), torch.uint8, w.device, stream)
            qT = _new((cols, rows), torch.uint8, w.device, stream) if transpose else None
            s = _new((rows // 128, cols // 128), torch.float32, w.device, stream)
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
    q = _new((rows, cols), torch.uint8, w.device, stream) if q is None else _dense(q, torch.uint8, "q")
    if transpose:
        qT = _new((cols, rows), torch.uint8, w.device, stream) if qT is None else _dense(qT, torch.uint8, "qT")
        _shape(qT, (cols, rows), "qT")
    else:
        qT = None
    s = _new((rows // 128, cols // 128), torch.float32, w.device, stream) if s is None else _dense(s, torch.float32, "s")
    _shape(q, (rows, cols), "q")
    _shape(s, (rows // 128, cols // 128), "s")
    _check(load_library().fp8_quantize_block(w.data_ptr(), rows, cols, w.stride(0), q.data_ptr(),
                                             qT.data_ptr() if qT is not None else None, s.data_ptr(),
                                             scale_mode, _stream(stream)))
    return q, qT, s


# ------------------------------------------------------------------- GEMMs --

def _out(shape, out_dtype, device, out, stream):
    if out is not None:
        return _shape(_dense(out, out_dtype, "out"), shape, "out")
    return _new(shape, out_dtype, device, stream)


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


def _operands(named, M, N, K):
    """Check each (tensor, name, role) of a contraction: codes are dense uint8
    and scales dense fp32 of exactly the shape the op's M, N, K imply.
    Roles: 'x' [M,K] + [M,K/128]; 'dy' [M,N] + [M,N/128]; 'w' [N,K] +
    [N/128,K/128] block scales; 'wT' [K,N]; 'dyT' [N,M] + [N,M/128];
    'xT' [K,M] + [K,M/128]."""
    import torch
    code_shape = {"x": (M, K), "dy": (M, N), "w": (N, K), "wT": (K, N), "dyT": (N, M), "xT": (K, M)}
    scale_shape = {"x": (M, K // 128), "dy": (M, N // 128), "w": (N // 128, K // 128),
                   "wT": (N // 128, K // 128), "dyT": (N, M // 128), "xT": (K, M // 128)}
    for codes, scales, role, name in named:
        _shape(_dense(codes, torch.uint8, name), code_shape[role], name)
        _shape(_dense(scales, torch.float32, name + " scales"), scale_shape[role], name + " scales")


def _workspace(op, M, N, K, workspace, device, stream):
    import torch
    need = fp8_block_gemm_workspace_size(op, M, N, K)
    if need and workspace is None:
        # belongs to `stream`: freed when this call returns, its memory is
        # reused only by work queued behind the kernels that use it
        workspace = _new(need, torch.uint8, device, stream)
    if workspace is None:
        return None, 0
    _dev(workspace, workspace.dtype, "workspace", ndim=workspace.dim())
    if not workspace.is_contiguous():
        raise ValueError("workspace: must be contiguous")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def fp8_block_gemm_workspace_size(op: int, M: int, N: int, K: int) -> int:
    return int(load_library().fp8_block_gemm_workspace_size(op, M, N, K))


# operand roles of (a, b) per op of the generic entry point, and the output shape
_GEMM_ROLES = {FP8BLK_OP_FPROP: ("x", "w"), FP8BLK_OP_DGRAD: ("dy", "wT"), FP8BLK_OP_WGRAD: ("dyT", "xT"),
               FP8BLK_OP_DGRAD_W: ("dy", "w")}


def fp8_block_gemm(op, a, sa, b, sb, M, N, K, out_dtype=None, algo=FP8BLK_ALGO_DEFAULT, out=None,
                   workspace=None, stream=None, accumulate=False, scale_mode=FP8BLK_SCALE_POW2):
    """Any of the three contractions with an explicit algorithm (see
    fp8_block_gemm in include/fp8blk.h for the operand roles).  accumulate:
    out += result in fp32 (out_dtype float32, `out` given).  scale_mode: the
    rule that made sa and sb (FP8BLK_SCALE_FP32 scales run PROMOTE)."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if op not in _GEMM_ROLES:
        raise ValueError(f"op {op}: not a contraction of fp8_block_gemm")
    ra, rb = _GEMM_ROLES[op]
    _operands(((a, sa, ra, "a"), (b, sb, rb, "b")), M, N, K)
    shape = {FP8BLK_OP_FPROP: (M, N), FP8BLK_OP_DGRAD: (M, K), FP8BLK_OP_WGRAD: (N, K), FP8BLK_OP_DGRAD_W: (M, K)}[op]
    y = _out(shape, out_dtype, a.device, out, stream)
    wptr, wbytes = _workspace(op, M, N, K, workspace, a.device, stream)
    _check(load_library().fp8_block_gemm(op, M, N, K, a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                                         y.data_ptr(), _odt(out_dtype, accumulate, out), algo, scale_mode, wptr,
                                         wbytes, _stream(stream)))
    return y


def fp8_block_gemm_fprop(qx, sx, qw, sw, out_dtype=None, out=None, stream=None, accumulate=False):
    """Y = X W^T.  qx [M,K], sx [M,K/128], qw [N,K], sw [N/128,K/128] -> Y [M,N]."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    M, K = qx.shape
    N = qw.shape[0]
    _operands(((qx, sx, "x", "qx"), (qw, sw, "w", "qw")), M, N, K)
    y = _out((M, N), out_dtype, qx.device, out, stream)
    _check(load_library().fp8_block_gemm_fprop(M, N, K, qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(),
                                               y.data_ptr(), _odt(out_dtype, accumulate, out), _stream(stream)))
    return y


def fp8_block_gemm_dgrad(qdy, sdy, qwT, sw, out_dtype=None, out=None, stream=None, accumulate=False):
    """dX = dY W.  qdy [M,N], sdy [M,N/128], qwT [K,N], sw [N/128,K/128] -> dX [M,K]."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    M, N = qdy.shape
    K = qwT.shape[0]
    _operands(((qdy, sdy, "dy", "qdy"), (qwT, sw, "wT", "qwT")), M, N, K)
    y = _out((M, K), out_dtype, qdy.device, out, stream)
    _check(load_library().fp8_block_gemm_dgrad(M, N, K, qdy.data_ptr(), sdy.data_ptr(), qwT.data_ptr(),
                                               sw.data_ptr(), y.data_ptr(), _odt(out_dtype, accumulate, out),
                                               _stream(stream)))
    return y


def fp8_block_gemm_dgrad_w(qdy, sdy, qw, sw, out_dtype=None, out=None, stream=None, accumulate=False):
    """dX = dY W from the weight codes as quantized.  qdy [M,N], sdy [M,N/128],
    qw [N,K], sw [N/128,K/128] -> dX [M,K]."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    M, N = qdy.shape
    K = qw.shape[1]
    _operands(((qdy, sdy, "dy", "qdy"), (qw, sw, "w", "qw")), M, N, K)
    y = _out((M, K), out_dtype, qdy.device, out, stream)
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
    _operands(((qdyT, sdyT, "dyT", "qdyT"), (qxT, sxT, "xT", "qxT")), M, N, K)
    y = _out((N, K), out_dtype, qdyT.device, out, stream)
    wptr, wbytes = _workspace(FP8BLK_OP_WGRAD, M, N, K, workspace, qdyT.device, stream)
    _check(load_library().fp8_block_gemm_wgrad(M, N, K, qdyT.data_ptr(), sdyT.data_ptr(), qxT.data_ptr(),
                                               sxT.data_ptr(), y.data_ptr(), _odt(out_dtype, accumulate, out), wptr,
                                               wbytes, _stream(stream)))
    return y


def fp8_block_gemm_backward(qdy, sdy, qwT, sw, qdyT, sdyT, qxT, sxT, dx_dtype=None, dw_dtype=None, dx=None,
                            dw=None, workspace=None, stream=None, accumulate_dw=False, scale_mode=FP8BLK_SCALE_POW2):
    """Dgrad and Wgrad of one linear in one call.  Operands as for
    fp8_block_gemm_dgrad and fp8_block_gemm_wgrad; returns (dx [M,K], dw [N,K]).
    accumulate_dw: dw += dY^T X in fp32 (dw_dtype float32, `dw` given).
    scale_mode: the rule that made the scales (FP8BLK_SCALE_FP32 runs PROMOTE)."""
    return _backward("fp8_block_gemm_backward", qdy, sdy, qwT, "wT", sw, qdyT, sdyT, qxT, sxT, dx_dtype,
                     dw_dtype, dx, dw, workspace, stream, accumulate_dw, scale_mode)


def fp8_block_gemm_backward_w(qdy, sdy, qw, sw, qdyT, sdyT, qxT, sxT, dx_dtype=None, dw_dtype=None, dx=None,
                              dw=None, workspace=None, stream=None, accumulate_dw=False, scale_mode=FP8BLK_SCALE_POW2):
    """fp8_block_gemm_backward with Dgrad reading the weight codes qw [N,K] as
    quantized (no transposed copy)."""
    return _backward("fp8_block_gemm_backward_w", qdy, sdy, qw, "w", sw, qdyT, sdyT, qxT, sxT, dx_dtype,
                     dw_dtype, dx, dw, workspace, stream, accumulate_dw, scale_mode)


def _backward(fn, qdy, sdy, wcodes, wrole, sw, qdyT, sdyT, qxT, sxT, dx_dtype, dw_dtype, dx, dw, workspace, stream,
              accumulate_dw, scale_mode):
    import torch
    dx_dtype = torch.bfloat16 if dx_dtype is None else dx_dtype
    dw_dtype = torch.bfloat16 if dw_dtype is None else dw_dtype
    M, N = qdy.shape
    K = wcodes.shape[1] if wrole == "w" else wcodes.shape[0]
    _operands(((qdy, sdy, "dy", "qdy"), (wcodes, sw, wrole, "weight codes"), (qdyT, sdyT, "dyT", "qdyT"),
               (qxT, sxT, "xT", "qxT")), M, N, K)
    x = _out((M, K), dx_dtype, qdy.device, dx, stream)
    w = _out((N, K), dw_dtype, qdy.device, dw, stream)
    wptr, wbytes = _workspace(FP8BLK_OP_BACKWARD, M, N, K, workspace, qdy.device, stream)
    _check(getattr(load_library(), fn)(M, N, K, qdy.data_ptr(), sdy.data_ptr(), wcodes.data_ptr(),
                                       sw.data_ptr(), qdyT.data_ptr(), sdyT.data_ptr(), qxT.data_ptr(),
                                       sxT.data_ptr(), x.data_ptr(), _odt(dx_dtype),
                                       w.data_ptr(), _odt(dw_dtype, accumulate_dw, dw), scale_mode, wptr, wbytes,
                                       _stream(stream)))
    return x, w


def fp8_block_gemm_backward_w_noalloc(qdy, sdy, qw, sw, qdyT, sdyT, qxT, sxT, dx, dw, stream=None,
                                      accumulate_dw=False, scale_mode=FP8BLK_SCALE_POW2):
    """fp8_block_gemm_backward_w for callers that cannot allocate: the
    library's static device scratch stands in for the workspace, and the
    outputs dx [M,K] and dw [N,K] (bf16 or fp32) must be given -- nothing is
    allocated, here or in the library.  Calls that overlap on one GPU share
    that scratch and race: order them on one stream.  Raises RuntimeError
    (FP8BLK_ERR_SCRATCH) if the launch would need more scratch than
    FP8BLK_NOALLOC_SCRATCH_BYTES."""
    import torch
    M, N = qdy.shape
    K = qw.shape[1]
    _operands(((qdy, sdy, "dy", "qdy"), (qw, sw, "w", "weight codes"), (qdyT, sdyT, "dyT", "qdyT"),
               (qxT, sxT, "xT", "qxT")), M, N, K)
    for t, name, shape in ((dx, "dx", (M, K)), (dw, "dw", (N, K))):
        if t is None:
            raise ValueError(f"{name}: the no-allocation call needs its outputs")
        if t.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError(f"{name}: bfloat16 or float32 expected")
        _shape(_dense(t, t.dtype, name), shape, name)
    _check(load_library().fp8_block_gemm_backward_w_noalloc(
        M, N, K, qdy.data_ptr(), sdy.data_ptr(), qw.data_ptr(), sw.data_ptr(), qdyT.data_ptr(), sdyT.data_ptr(),
        qxT.data_ptr(), sxT.data_ptr(), dx.data_ptr(), _odt(dx.dtype), dw.data_ptr(),
        _odt(dw.dtype, accumulate_dw, dw), scale_mode, _stream(stream)))
    return dx, dw
