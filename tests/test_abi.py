"""The C ABI, checked without a GPU: the library loads, exports every
function include/fp8blk.h declares, and every host-side argument check
returns its documented status before anything is launched (the pointers
below are never dereferenced: each call fails validation first)."""
import ctypes
import os
import shutil
import subprocess

import pytest

import blockwise_fp8_linear_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, ENULL, EDIM, EALIGN, EARG, EWS, EHIP, EDEV, ESCR = 0, -1, -2, -3, -4, -5, -6, -7, -8
P = 0x100000          # a fake, 16-byte aligned device address (never used)
P2 = 0x200000
P3 = 0x300000
MIS = 0x100008        # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    return fb.load_library()


def test_exports_every_declared_function(lib):
    names = fb.header_functions()
    assert set(names) == {
        "fp8_quantize_rowgroup", "fp8_quantize_colgroup", "fp8_quantize_block", "fp8_quantize_dual",
        "fp8_quantize_block_batch",
        "fp8_block_gemm_fprop", "fp8_block_gemm_dgrad", "fp8_block_gemm_wgrad", "fp8_block_gemm_backward",
        "fp8_block_gemm_dgrad_w", "fp8_block_gemm_backward_w", "fp8_block_gemm_backward_w_noalloc",
        "fp8_block_gemm", "fp8_block_gemm_workspace_size", "fp8_status_string",
    }
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for rc in (OK, ENULL, EDIM, EALIGN, EARG, EWS, EHIP, EDEV, ESCR):
        assert fb.fp8_status_string(rc)
    assert "unknown" in fb.fp8_status_string(-99)


def test_rowgroup_errors(lib):
    f = lib.fp8_quantize_rowgroup
    assert f(P, 4, 256, 256, P2, 256, P3, 2, None) == EARG      # scale mode (0 and 1 are valid)
    assert f(P, 4, 256, 256, P2, 256, P3, -1, None) == EARG
    assert f(P, 4, 256, 256, P2, 256, P3, 1, None) in (EHIP, EDEV)   # amax / 448 scales: valid
    assert f(None, 4, 256, 256, P2, 256, P3, 0, None) == ENULL
    assert f(P, 4, 256, 256, None, 256, P3, 0, None) == ENULL
    assert f(P, 4, 256, 256, P2, 256, None, 0, None) == ENULL
    assert f(P, 0, 256, 256, P2, 256, P3, 0, None) == EDIM      # empty
    assert f(P, 4, 200, 256, P2, 256, P3, 0, None) == EDIM      # ragged cols
    assert f(P, 4, 0, 256, P2, 256, P3, 0, None) == EDIM
    assert f(P, 4, 256, 128, P2, 256, P3, 0, None) == EARG      # ld < cols
    assert f(P, 4, 256, 256, P2, 128, P3, 0, None) == EARG
    assert f(MIS, 4, 256, 256, P2, 256, P3, 0, None) == EALIGN
    assert f(P, 4, 256, 260, P2, 256, P3, 0, None) == EALIGN    # ld_x not a multiple of 8
    assert f(P, 4, 256, 256, P2, 264, P3, 0, None) == EALIGN    # ld_q not a multiple of 16
    assert f(P, 4, 256, 256, P2, 256, P3 + 2, 0, None) == EALIGN


def test_size_limits_without_overflow(lib):
    """Sizes whose products overflow 64 bits, or exceed what the kernels'
    index arithmetic covers, are rejected with FP8BLK_ERR_ARG."""
    big = 1 << 40                                                      # a multiple of 128
    huge = 1 << 61
    assert lib.fp8_quantize_rowgroup(P, huge, 128, 128, P2, 128, P3, 0, None) == EARG
    assert lib.fp8_quantize_rowgroup(P, 1 << 20, big, big, P2, big, P3, 0, None) == EARG
    assert lib.fp8_quantize_rowgroup(P, 4, 256, huge, P2, 256, P3, 0, None) == EARG   # ld_x too large
    assert lib.fp8_quantize_colgroup(P, big, big, big, P2, big, P3, 0, None) == EARG
    assert lib.fp8_quantize_dual(P, big, big, big, P2, big, P3, P2, big, P3, 0, None) == EARG
    assert lib.fp8_quantize_block(P, big, big, big, P2, None, P3, 0, None) == EARG
    f = lib.fp8_block_gemm_fprop
    assert f(huge, huge, 256, P, P3, P2, P3, P, 0, None) == EARG
    assert f(1 << 26, 1 << 26, 1 << 26, P, P3, P2, P3, P, 0, None) == EARG            # M * N > 2^40
    assert lib.fp8_block_gemm_backward(huge, 256, 256, P, P3, P2, P3, P, P3, P2, P3, P, 0, P + 64, 0, 0,
                                       None, 0, None) == EARG


def test_colgroup_and_block_errors(lib):
    f = lib.fp8_quantize_colgroup
    assert f(P, 200, 256, 256, P2, 256, P3, 0, None) == EDIM    # rows must be a multiple of 128
    assert f(P, 256, 256, 256, P2, 128, P3, 0, None) == EARG    # ld_qT < rows
    assert f(None, 256, 256, 256, P2, 256, P3, 0, None) == ENULL
    assert f(P, 256, 256, 256, MIS, 256, P3, 0, None) == EALIGN
    g = lib.fp8_quantize_block
    assert g(P, 256, 384, 384, P2, None, P3, 0, None) != ENULL  # qT may be NULL (fails later: no GPU)
    assert g(P, 256, 300, 384, P2, None, P3, 0, None) == EDIM
    assert g(P, 256, 384, 256, P2, None, P3, 0, None) == EARG
    assert g(P, 256, 384, 384, P2, MIS, P3, 0, None) == EALIGN
    assert g(P, 256, 384, 384, P2, None, P3, 7, None) == EARG


def test_dual_errors(lib):
    f = lib.fp8_quantize_dual
    P4, P5 = 0x400000, 0x500000
    ok = (P, 256, 384, 384, P2, 384, P3, P4, 256, P5, 0, None)
    assert f(*ok) in (EHIP, EDEV)                                 # valid arguments, no GPU here

    def call(**kw):
        names = ("x", "rows", "cols", "ld_x", "q", "ld_q", "s", "qT", "ld_qT", "sT", "mode", "stream")
        a = dict(zip(names, ok))
        a.update(kw)
        return f(*[a[n] for n in names])
    assert call(mode=2) == EARG
    assert call(mode=1) in (EHIP, EDEV)
    for n in ("x", "q", "s", "qT", "sT"):
        assert call(**{n: None}) == ENULL, n
    assert call(rows=200) == EDIM                                 # both dims multiples of 128
    assert call(cols=200, ld_x=256, ld_q=256) == EDIM
    assert call(rows=0) == EDIM
    assert call(ld_x=256) == EARG                                 # ld < cols
    assert call(ld_q=256) == EARG
    assert call(ld_qT=128) == EARG                                # ld_qT < rows
    assert call(x=MIS) == EALIGN
    assert call(qT=MIS) == EALIGN
    assert call(sT=P5 + 2) == EALIGN
    assert call(ld_x=388) == EALIGN                               # not a multiple of 8
    assert call(ld_qT=264) == EALIGN                              # not a multiple of 16


def test_block_batch_errors(lib):
    J = fb._BlockJob
    good = [J(P, 256, 384, 384, P2, None, P3), J(P, 512, 128, 128, P2, P2 + 0x10000, P3)]
    arr = lambda jobs: (J * len(jobs))(*jobs)
    assert lib.fp8_quantize_block_batch(arr(good), 2, 0, None) in (EHIP, EDEV)   # valid, no GPU here
    assert lib.fp8_quantize_block_batch(None, 1, 0, None) == ENULL
    assert lib.fp8_quantize_block_batch(arr(good), 0, 0, None) == EARG
    assert lib.fp8_quantize_block_batch(arr(good * 5), 9, 0, None) == EARG        # at most 8 jobs
    assert lib.fp8_quantize_block_batch(arr(good), 2, 2, None) == EARG            # scale mode
    assert lib.fp8_quantize_block_batch(arr(good), 2, 1, None) in (EHIP, EDEV)
    bad = [good[0], J(P, 256, 300, 384, P2, None, P3)]
    assert lib.fp8_quantize_block_batch(arr(bad), 2, 0, None) == EDIM             # second job's shape
    bad = [good[0], J(P, 256, 384, 384, None, None, P3)]
    assert lib.fp8_quantize_block_batch(arr(bad), 2, 0, None) == ENULL
    bad = [J(MIS, 256, 384, 384, P2, None, P3)]
    assert lib.fp8_quantize_block_batch(arr(bad), 1, 0, None) == EALIGN


def test_gemm_errors(lib):
    f = lib.fp8_block_gemm_fprop
    assert f(256, 256, 256, P, P3, P2, P3, P, 5, None) == EARG           # out dtype
    assert f(256, 256, 256, P, P3, P2, P3, P, 3, None) == EARG
    assert f(256, 256, 256, P, P3, P2, P3, P, 2, None) in (EHIP, EDEV)  # fp32 accumulate: valid
    assert f(256, 256, 256, None, P3, P2, P3, P, 0, None) == ENULL
    assert f(256, 256, 256, P, P3, P2, None, P, 0, None) == ENULL
    assert f(256, 200, 256, P, P3, P2, P3, P, 0, None) == EDIM
    assert f(0, 256, 256, P, P3, P2, P3, P, 0, None) == EDIM
    assert f(256, 256, 256, MIS, P3, P2, P3, P, 0, None) == EALIGN
    assert f(256, 256, 256, P, P3 + 1, P2, P3, P, 0, None) == EALIGN
    g = lib.fp8_block_gemm
    assert g(3, 256, 256, 256, P, P3, P2, P3, P, 0, 0, 0, None, 0, None) == EARG   # op
    assert g(5, 256, 256, 256, P, P3, P2, P3, P, 0, 0, 0, None, 0, None) == EARG
    assert g(4, 256, 256, 256, P, P3, P2, P3, P, 0, 1, 0, None, 0, None) in (EHIP, EDEV)   # Dgrad from qw
    assert lib.fp8_block_gemm_workspace_size(4, 8192, 2048, 2048) == lib.fp8_block_gemm_workspace_size(1, 8192, 2048, 2048)
    d = lib.fp8_block_gemm_dgrad_w
    assert d(256, 256, 256, P, P3, P2, P3, P, 0, None) in (EHIP, EDEV)
    assert d(256, 256, 256, P, P3, None, P3, P, 0, None) == ENULL
    assert d(256, 200, 256, P, P3, P2, P3, P, 0, None) == EDIM
    assert d(256, 256, 256, P, P3, MIS, P3, P, 0, None) == EALIGN
    assert d(256, 256, 256, P, P3, P2, P3, P, 4, None) == EARG
    assert g(0, 256, 256, 256, P, P3, P2, P3, P, 0, 9, 0, None, 0, None) == EARG   # algo
    # wgrad at a shape that splits the reduction needs a workspace
    need = lib.fp8_block_gemm_workspace_size(2, 8192, 256, 256)
    assert need > 0
    w = lib.fp8_block_gemm_wgrad
    assert w(8192, 256, 256, P, P3, P2, P3, P, 0, None, 0, None) == EWS
    assert w(8192, 256, 256, P, P3, P2, P3, P, 0, P, need - 1, None) == EWS
    assert w(8192, 256, 256, P, P3, P2, P3, P, 0, MIS, need, None) == EALIGN


@pytest.mark.parametrize("fn", ["fp8_block_gemm_backward", "fp8_block_gemm_backward_w"])
def test_backward_errors(lib, fn):
    f = getattr(lib, fn)
    P4, P5, P6, P7 = 0x400000, 0x500000, 0x600000, 0x700000
    need = lib.fp8_block_gemm_workspace_size(3, 8192, 2048, 2048)
    assert need > 0 and need != ctypes.c_size_t(-1).value
    names = ("M", "N", "K", "qdy", "sdy", "qwT", "sw", "qdyT", "sdyT", "qxT", "sxT", "dx", "dxt", "dw", "dwt",
             "mode", "ws", "wsb", "stream")
    ok = (8192, 2048, 2048, P, P3, P2, P3, P4, P5, P6, P7, 0x800000, 0, 0x900000, 1, 0, 0xA00000, need, None)

    def call(**kw):
        a = dict(zip(names, ok))
        a.update(kw)
        return f(*[a[n] for n in names])
    assert call() in (EHIP, EDEV)                                  # valid arguments, no GPU here
    assert call(dxt=2) in (EHIP, EDEV)                             # fp32 accumulate allowed
    assert call(dwt=7) == EARG
    assert call(dx=0x900000) == EARG                               # dx and dw alias
    for n in ("qdy", "sdy", "qwT", "sw", "qdyT", "sdyT", "qxT", "sxT", "dx", "dw"):
        assert call(**{n: None}) == ENULL, n
    assert call(N=200) == EDIM
    assert call(ws=None) == EWS
    assert call(wsb=need - 1) == EWS
    assert call(ws=MIS) == EALIGN
    assert call(qxT=MIS) == EALIGN


@pytest.mark.parametrize("op", [0, 1, 2, 4])
def test_gemm_scale_mode(lib, op):
    """amax / 448 scales are not powers of two: the block-scaled MFMA would
    keep only their exponent bits, so that pairing is refused before any
    launch, DEFAULT resolves to PROMOTE (valid: fails later, on the device
    check), and an unknown scale mode is refused."""
    g = lib.fp8_block_gemm
    need = lib.fp8_block_gemm_workspace_size(op, 8192, 2048, 2048)
    ws = P if need else None
    args = lambda algo, mode: (op, 8192, 2048, 2048, P, P3, P2, P3, P, 0, algo, mode, ws, need, None)
    assert g(*args(2, 1)) == EARG                       # SCALED_MFMA with amax / 448 scales
    for algo in (0, 1):                                 # DEFAULT (-> PROMOTE) and PROMOTE: valid
        assert g(*args(algo, 1)) in (EHIP, EDEV)
    for algo in (0, 1, 2):                              # power-of-two scales: every algorithm
        assert g(*args(algo, 0)) in (EHIP, EDEV)
    for mode in (-1, 2, 7):
        assert g(*args(0, mode)) == EARG


@pytest.mark.parametrize("fn", ["fp8_block_gemm_backward", "fp8_block_gemm_backward_w"])
def test_backward_scale_mode(lib, fn):
    f = getattr(lib, fn)
    need = lib.fp8_block_gemm_workspace_size(3, 8192, 2048, 2048)
    args = lambda mode: (8192, 2048, 2048, P, P3, P2, P3, 0x400000, 0x500000, 0x600000, 0x700000, 0x800000, 0,
                         0x900000, 1, mode, 0xA00000, need, None)
    assert f(*args(0)) in (EHIP, EDEV)
    assert f(*args(1)) in (EHIP, EDEV)                  # amax / 448: the promote algorithm
    for mode in (-1, 2):
        assert f(*args(mode)) == EARG


def test_noalloc_backward_host_checks(lib):
    """The no-allocation backward: argument errors as for the workspace form,
    and a launch that would need more than the static scratch is refused
    before anything runs (the fused launch at 1536 x 1536 x 2560 cuts its
    ranges into 288 partial 256x256 tiles: 72 MiB)."""
    f = lib.fp8_block_gemm_backward_w_noalloc
    args = lambda M, N, K, mode, dx=0x800000, dw=0x900000: (M, N, K, P, P3, P2, P3, 0x400000, 0x500000, 0x600000,
                                                            0x700000, dx, 0, dw, 1, mode, None)
    assert f(*args(8192, 2048, 2048, 0)) in (EHIP, EDEV)       # fused launch, 32 MiB of slots: fits
    assert f(*args(8192, 2048, 6144, 0)) in (EHIP, EDEV)
    assert f(*args(8192, 2048, 6144, 1)) in (EHIP, EDEV)       # promote pair: 32 MiB of Wgrad partials
    assert f(*args(1536, 1536, 2560, 0)) == ESCR               # needs 72 MiB > 64 MiB
    assert f(*args(8192, 2048, 2048, 2)) == EARG
    assert f(*args(8192, 2048, 2048, 0, dx=0x900000)) == EARG  # dx and dw alias
    assert f(*args(8192, 200, 2048, 0)) == EDIM
    assert f(*args(8192, 2048, 2048, 0, dx=None)) == ENULL
    assert "scratch" in fb.fp8_status_string(ESCR)


def test_workspace_query(lib):
    q = lib.fp8_block_gemm_workspace_size
    assert q(0, 8192, 12288, 2048) == 0                 # fprop never needs one
    assert q(1, 8192, 4096, 2048) == 0
    assert q(2, 100, 256, 256) == ctypes.c_size_t(-1).value
    assert q(7, 256, 256, 256) == ctypes.c_size_t(-1).value
    # O-projection wgrad: 64 output tiles of 256x256 whose 8192-token
    # reduction (16 units of 512) is cut into 4 pieces each by the 256
    # workgroups: one 256x256 fp32 slot per partial segment (256 of them),
    # and at least what the general kernel's stream-K partials need (256 of
    # its 256x128 tiles)
    n = q(2, 8192, 2048, 2048)
    assert n == max(256 * 256 * 256 * 4, 2 * 2048 * 2048 * 4)
    # the fused backward of the same linear: Dgrad's 256 tiles fall whole
    # into ranges, Wgrad's 64 tiles are cut in two -- 128 partial segments
    assert q(3, 8192, 2048, 2048) == max(128 * 256 * 256 * 4, n)
    # a 512-token reduction is one unit per tile: no tile is shared
    assert q(2, 512, 5120, 7680) == 0
    # dimensions the GEMM entry points reject are invalid shapes here too
    big = 128 << 20
    for op in (0, 1, 2, 3, 4):
        assert q(op, big, 256, 256) == ctypes.c_size_t(-1).value
        assert q(op, 256, 256, big) == ctypes.c_size_t(-1).value


def test_valid_call_without_gpu_reports_device_error(lib):
    """With valid arguments the only remaining check is the device; on a
    machine without a gfx950 it must fail cleanly, never launch."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc = lib.fp8_quantize_rowgroup(P, 4, 256, 256, P2, 256, P3, 0, None)
    assert rc in (EHIP, EDEV)
    rc = lib.fp8_block_gemm_fprop(256, 256, 256, P, P3, P2, P3, P, 0, None)
    assert rc in (EHIP, EDEV)


def test_binding_fails_loudly_when_library_missing(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        fb._lib = None
        try:
            fb.load_library(str(tmp_path / "nope.so"))
        finally:
            fb._lib = None


def test_probe_library():
    """The measurement probe (include/fp8probe.h) loads, counts its FLOPs, and
    rejects bad arguments before launching."""
    from blockwise_fp8_linear_amd.build import PROBE_LIB
    p = ctypes.CDLL(PROBE_LIB)
    p.fp8probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    p.fp8probe_mfma_flops.restype = ctypes.c_double
    assert p.fp8probe_mfma_flops(256, 10) == 256 * 10 * 4 * 16 * 2 * 32 * 32 * 64
    p.fp8probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    assert p.fp8probe_mfma(0, 10, 1, P, None) == -1
    assert p.fp8probe_mfma(256, 0, 1, P, None) == -1
    assert p.fp8probe_mfma(256, 10, 1, None, None) == -1
    p.fp8probe_pow2_cvt_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert p.fp8probe_pow2_cvt_check(None, None) == -1
    p.fp8probe_fp32_quotient_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert p.fp8probe_fp32_quotient_check(None, None) == -1


def test_c_program_against_the_header(tmp_path):
    """include/fp8blk.h compiles as strict C99, every entry point links, and
    each rejects a bad argument with the documented status (no GPU needed:
    no call reaches the device)."""
    if shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no gcc or no HIP headers")
    libdir = os.path.dirname(fb.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-isystem", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "abi_from_c.c"), "-o", exe,
                    "-L", libdir, "-l:libfp8blk.so", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
