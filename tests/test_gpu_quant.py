"""GPU parity of the three quantizers against the CPU oracle: codes and
scales must be bit-exact.  Inputs are the seeded synthetic workloads (the
tiny fprop case, the 8192-token gate/up linear, the decoder-layer shapes, the
outlier-stress variant) plus constructed edge tensors: ragged row counts,
strided column slices, all-zero groups, bf16-subnormal groups and an
exhaustive sweep of the cast over every bf16 magnitude at every scale."""
import numpy as np
import pytest

import oracle
from blockwise_fp8_linear_amd import synth
from gpu_util import dev, dev_bf16, host, note, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _rowgroup(x_bits, cols=None, mode=0):
    import torch
    import blockwise_fp8_linear_amd as fb
    xt = dev_bf16(x_bits)
    if cols is not None:
        xt = xt[:, :cols]
    q, s = fb.fp8_quantize_rowgroup(xt, scale_mode=mode)
    torch.cuda.synchronize()
    return host(q), host(s)


def _assert_rowgroup(x_bits, what, cols=None, mode=0):
    note(f"rowgroup {what} {x_bits.shape} cols={cols} mode={mode}")
    q, s = _rowgroup(x_bits, cols, mode)
    q0, s0 = oracle.quantize_rowgroup(x_bits, cols=cols, mode=mode)
    assert np.array_equal(s, s0), f"{what}: scales differ ({int((s != s0).sum())})"
    assert np.array_equal(q, q0), f"{what}: codes differ ({int((q != q0).sum())})"


def test_rowgroup_tiny_and_ragged_rows():
    x, _ = synth.tiny_fprop()
    _assert_rowgroup(x, "tiny X")
    for rows in (1, 3, 17, 257):
        _assert_rowgroup(synth.normal_bf16((rows, 384), 1.0, 40, rows), f"ragged rows={rows}")


def test_rowgroup_single_linear_x():
    x, _ = synth.single_linear()
    _assert_rowgroup(x, "8192x2048 X")


def test_rowgroup_outlier_stress():
    x, _, info = synth.outlier_stress()
    _assert_rowgroup(x, "outlier X")


def test_rowgroup_column_slice_and_padded_output():
    import torch
    import blockwise_fp8_linear_amd as fb
    wide = synth.normal_bf16((512, 4096), 1.0, 41, 0)
    _assert_rowgroup(wide, "column slice", cols=2048)
    # output with a row stride larger than cols
    xt = dev_bf16(wide)[:, :1024]
    qbuf = torch.full((512, 1536), 0xAB, dtype=torch.uint8, device="cuda")
    q, s = fb.fp8_quantize_rowgroup(xt, q=qbuf[:, :1024])
    torch.cuda.synchronize()
    q0, s0 = oracle.quantize_rowgroup(wide, cols=1024)
    qh = host(qbuf)
    assert np.array_equal(qh[:, :1024], q0) and np.array_equal(host(s), s0)
    assert np.all(qh[:, 1024:] == 0xAB)          # nothing written past cols


def test_rowgroup_decoder_layer_gradients():
    for lin in synth.decoder_layer():
        _assert_rowgroup(lin["dy"], f"dY {lin['name']}")


def test_rowgroup_exhaustive_cast():
    """Every non-negative bf16 magnitude up to 448 (and its negative) placed
    in groups whose amax is exactly 448 * 2^e, for every e in [-126, 118]:
    the kernel must reproduce the oracle on every element."""
    mags = (np.arange(0x8000, dtype=np.uint32) << 16).view(np.float32)
    mags = mags[np.isfinite(mags) & (mags <= 448.0)]
    vals = np.concatenate([mags, -mags]).astype(np.float32)
    per = 127
    ng = (vals.size + per - 1) // per
    vals = np.concatenate([vals, np.zeros(ng * per - vals.size, np.float32)]).reshape(ng, per)
    es = np.arange(-126, 119)
    rows = []
    for e in es:
        blk = np.empty((ng, 128), np.float32)
        blk[:, 0] = 448.0 * np.float32(2.0 ** e)
        blk[:, 1:] = vals * np.float32(2.0 ** e)
        rows.append(blk)
    x = synth.bf16_bits_from_f32(np.concatenate(rows).reshape(-1, 128))
    _assert_rowgroup(x, "exhaustive cast")


def test_rowgroup_edge_groups():
    x = synth.normal_bf16((256, 1024), 1.0, 42, 0)
    x[3, 128:256] = 0                                            # all +0
    x[4, :128] = 0x8000                                          # all -0
    x[5, 256:384] = np.arange(128, dtype=np.uint16)              # bf16 subnormals
    x[6, 384:512] = (np.arange(128, dtype=np.uint16) | 0x8000)   # negative subnormals
    x[7, :128] = synth.bf16_bits_from_f32(np.full(128, 3.0e38, np.float32))   # near bf16 max
    x[8, :128] = synth.bf16_bits_from_f32(np.linspace(-1e-30, 1e-30, 128).astype(np.float32))
    _assert_rowgroup(x, "edge groups")


def _colgroup(x_bits, mode=0):
    import torch
    import blockwise_fp8_linear_amd as fb
    qT, sT = fb.fp8_quantize_colgroup(dev_bf16(x_bits), scale_mode=mode)
    torch.cuda.synchronize()
    return host(qT), host(sT)


def _assert_colgroup(x_bits, what, mode=0):
    note(f"colgroup {what} {x_bits.shape} mode={mode}")
    qT, sT = _colgroup(x_bits, mode)
    q0, s0 = oracle.quantize_colgroup(x_bits, mode=mode)
    assert np.array_equal(sT, s0), f"{what}: scales differ ({int((sT != s0).sum())})"
    assert np.array_equal(qT, q0), f"{what}: codes differ ({int((qT != q0).sum())})"


def test_colgroup_small_and_edges():
    _assert_colgroup(synth.normal_bf16((128, 64 * 3), 1.0, 43, 0)[:, :128], "128x128")
    x = synth.normal_bf16((384, 640), 1.0, 43, 1)
    x[128:256, 5] = 0
    x[:128, 7] = np.arange(128, dtype=np.uint16)
    _assert_colgroup(x, "384x640 edges")


def test_colgroup_decoder_layer():
    for lin in synth.decoder_layer():
        _assert_colgroup(lin["x"], f"X {lin['name']}")
        _assert_colgroup(lin["dy"], f"dY {lin['name']}")


def test_colgroup_strided_input():
    import torch
    import blockwise_fp8_linear_amd as fb
    wide = synth.normal_bf16((1024, 4096), 1.0, 44, 0)
    qT, sT = fb.fp8_quantize_colgroup(dev_bf16(wide)[:, :2048])
    torch.cuda.synchronize()
    q0, s0 = oracle.quantize_colgroup(wide, cols=2048)
    assert np.array_equal(host(qT), q0) and np.array_equal(host(sT), s0)


def _assert_block(w_bits, what, transpose=True, mode=0):
    import torch
    import blockwise_fp8_linear_amd as fb
    note(f"block {what} {w_bits.shape} transpose={transpose} mode={mode}")
    q, qT, s = fb.fp8_quantize_block(dev_bf16(w_bits), transpose=transpose, scale_mode=mode)
    torch.cuda.synchronize()
    q0, qT0, s0 = oracle.quantize_block(w_bits, transpose=transpose, mode=mode)
    assert np.array_equal(host(s), s0), f"{what}: scales differ"
    assert np.array_equal(host(q), q0), f"{what}: codes differ"
    if transpose:
        assert np.array_equal(host(qT), qT0), f"{what}: transposed codes differ"


def test_block_tiny_and_edges():
    _, w = synth.tiny_fprop()
    _assert_block(w, "tiny W")
    w = synth.normal_bf16((384, 256), 0.02, 45, 0)
    w[128:256, 128:256] = 0
    w[:128, :128] = np.arange(128 * 128, dtype=np.uint16).reshape(128, 128) % 128   # subnormal block
    _assert_block(w, "edges")
    _assert_block(w, "edges, no transpose", transpose=False)


def test_block_single_linear_w():
    _, w = synth.single_linear()
    _assert_block(w, "12288x2048 W")


def test_block_decoder_layer():
    for lin in synth.decoder_layer():
        _assert_block(lin["w"], f"W {lin['name']}")


def _assert_dual(x_bits, what, cols=None, pad_q=0, pad_qT=0, mode=0):
    """The one-pass quantizer against the oracle's row-group and column-group
    quantizers, bit for bit; optional strided input and padded outputs (the
    padding must stay untouched)."""
    import torch
    import blockwise_fp8_linear_amd as fb
    note(f"dual {what} {x_bits.shape} cols={cols} pad={pad_q},{pad_qT} mode={mode}")
    xt = dev_bf16(x_bits)
    if cols is not None:
        xt = xt[:, :cols]
    rows, c = xt.shape
    qbuf = torch.full((rows, c + pad_q), 0xAB, dtype=torch.uint8, device="cuda")
    qTbuf = torch.full((c, rows + pad_qT), 0xCD, dtype=torch.uint8, device="cuda")
    q, s, qT, sT = fb.fp8_quantize_dual(xt, q=qbuf[:, :c], qT=qTbuf[:, :rows], scale_mode=mode)
    torch.cuda.synchronize()
    q0, s0 = oracle.quantize_rowgroup(x_bits, cols=cols, mode=mode)
    qT0, sT0 = oracle.quantize_colgroup(x_bits, cols=cols, mode=mode)
    qh, qTh = host(qbuf), host(qTbuf)
    assert np.array_equal(host(s), s0), f"{what}: row scales differ ({int((host(s) != s0).sum())})"
    assert np.array_equal(qh[:, :c], q0), f"{what}: row codes differ ({int((qh[:, :c] != q0).sum())})"
    assert np.array_equal(host(sT), sT0), f"{what}: column scales differ ({int((host(sT) != sT0).sum())})"
    assert np.array_equal(qTh[:, :rows], qT0), f"{what}: column codes differ ({int((qTh[:, :rows] != qT0).sum())})"
    assert np.all(qh[:, c:] == 0xAB) and np.all(qTh[:, rows:] == 0xCD), f"{what}: wrote past the end"


def test_dual_small_and_edges():
    x, _ = synth.tiny_fprop()
    _assert_dual(x, "tiny X")
    x = synth.normal_bf16((384, 640), 1.0, 47, 0)
    x[3, 128:256] = 0                                            # zero row group
    x[128:256, 5] = 0                                            # zero column group
    x[:128, 7] = np.arange(128, dtype=np.uint16)                 # subnormal column group
    x[200, 256:384] = (np.arange(128, dtype=np.uint16) | 0x8000)  # subnormal row group
    x[300, :128] = synth.bf16_bits_from_f32(np.full(128, 3.0e38, np.float32))
    x[256:384, 639] = synth.bf16_bits_from_f32(np.full(128, -3.0e38, np.float32))
    _assert_dual(x, "384x640 edges")


def test_dual_exhaustive_cast_both_orientations():
    """The exhaustive cast sweep of the row-group test, padded to whole
    tiles, through both the row-group side (as is) and the column-group side
    (transposed)."""
    mags = (np.arange(0x8000, dtype=np.uint32) << 16).view(np.float32)
    mags = mags[np.isfinite(mags) & (mags <= 448.0)]
    vals = np.concatenate([mags, -mags]).astype(np.float32)
    per = 127
    ng = (vals.size + per - 1) // per
    vals = np.concatenate([vals, np.zeros(ng * per - vals.size, np.float32)]).reshape(ng, per)
    blocks = []
    for e in range(-126, 119, 3):
        blk = np.empty((ng, 128), np.float32)
        blk[:, 0] = 448.0 * np.float32(2.0 ** e)
        blk[:, 1:] = vals * np.float32(2.0 ** e)
        blocks.append(blk)
    x = np.concatenate(blocks).reshape(-1, 128)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 128, 128), np.float32)])
    xb = synth.bf16_bits_from_f32(x)
    _assert_dual(xb, "exhaustive cast, row side")
    _assert_dual(np.ascontiguousarray(xb.T), "exhaustive cast, column side")


def test_dual_strided_input_padded_outputs():
    wide = synth.normal_bf16((1024, 4096), 1.0, 48, 0)
    _assert_dual(wide, "column slice, padded outputs", cols=2048, pad_q=256, pad_qT=128)


def test_dual_blocked_order_strided_padded():
    """A shape the one-pass quantizer walks in XCD blocks of 8 x 16 tiles
    (16 row tiles, 64 column tiles), read from a column slice of a wider
    tensor into padded outputs: every tile is written, bit for bit, and
    nothing past the outputs' ends."""
    wide = synth.normal_bf16((2048, 8192 + 256), 1.0, 49, 0)
    _assert_dual(wide, "blocked order, column slice, padded outputs", cols=8192, pad_q=128, pad_qT=256)


def test_dual_decoder_layer():
    for lin in synth.decoder_layer():
        _assert_dual(lin["x"], f"X {lin['name']}")
        _assert_dual(lin["dy"], f"dY {lin['name']}")


def test_dual_outlier_stress():
    x, _, _ = synth.outlier_stress()
    _assert_dual(x, "outlier X")


@pytest.mark.parametrize("mode", [0, 1])
def test_block_batch_equals_single(mode):
    """The batched block quantizer on the decoder layer's four weights (plus
    an edge-case weight without the transposed copy): each result bit-equal
    to the oracle, under both scale rules."""
    import torch
    import blockwise_fp8_linear_amd as fb
    ws = [lin["w"] for lin in synth.decoder_layer()]
    e = synth.normal_bf16((384, 256), 0.02, 45, 0)
    e[128:256, 128:256] = 0
    e[:128, :128] = np.arange(128 * 128, dtype=np.uint16).reshape(128, 128) % 128
    ws.append(e)
    note(f"block batch {[w.shape for w in ws]} mode={mode}")
    dev = [dev_bf16(w) for w in ws]
    res = (fb.fp8_quantize_block_batch(dev[:4], scale_mode=mode) +
           fb.fp8_quantize_block_batch(dev[4:], transpose=False, scale_mode=mode))
    torch.cuda.synchronize()
    for k, (w, (q, qT, s)) in enumerate(zip(ws, res)):
        q0, qT0, s0 = oracle.quantize_block(w, transpose=qT is not None, mode=mode)
        assert np.array_equal(host(s), s0), f"job {k}: scales differ"
        assert np.array_equal(host(q), q0), f"job {k}: codes differ"
        if qT is not None:
            assert np.array_equal(host(qT), qT0), f"job {k}: transposed codes differ"


def test_quantizers_repeatable():
    import torch
    import blockwise_fp8_linear_amd as fb
    x = dev_bf16(synth.normal_bf16((2048, 2048), 1.0, 46, 0))
    a = [fb.fp8_quantize_rowgroup(x), fb.fp8_quantize_colgroup(x), fb.fp8_quantize_block(x)[::2],
         fb.fp8_quantize_dual(x)]
    b = [fb.fp8_quantize_rowgroup(x), fb.fp8_quantize_colgroup(x), fb.fp8_quantize_block(x)[::2],
         fb.fp8_quantize_dual(x)]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        for s, t in zip(u, v):
            assert torch.equal(s, t)


# ---------------------------------------------------------------------------
# The amax / 448 scale rule (FP8BLK_SCALE_FP32, oracle mode 1): the same
# bit-exact bar.  Its scales are not powers of two, so every quotient x / s
# is a rounded IEEE division on both sides.

FP32 = 1


def _division_sweep():
    """Groups whose amax is a * 2^e for a few non-power-of-two mantissas a
    (so s = a * 2^e / 448 is inexact), the other 127 elements sweeping every
    bf16 magnitude up to a, and its negative, scaled alike; e across the
    exponent range, down to bf16 subnormal groups."""
    mags_all = (np.arange(0x8000, dtype=np.uint32) << 16).view(np.float32)
    blocks = []
    for a in (1.0, 1.375, 3.0, 300.0):
        mags = mags_all[np.isfinite(mags_all) & (mags_all <= a)]
        vals = np.concatenate([mags, -mags]).astype(np.float32)
        per = 127
        ng = (vals.size + per - 1) // per
        vals = np.concatenate([vals, np.zeros(ng * per - vals.size, np.float32)]).reshape(ng, per)
        for e in (-140, -128, -100, -37, -9, 0, 7, 50, 110):
            blk = np.empty((ng, 128), np.float32)
            blk[:, 0] = np.float32(a) * np.float32(2.0 ** e)
            blk[:, 1:] = vals * np.float32(2.0 ** e)
            blocks.append(blk)
    x = np.concatenate(blocks)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 128, 128), np.float32)])
    return synth.bf16_bits_from_f32(x)


def test_fp32_scale_rowgroup_edges_and_ragged():
    x = synth.normal_bf16((256, 1024), 1.0, 42, 0)
    x[3, 128:256] = 0                                            # all +0
    x[4, :128] = 0x8000                                          # all -0
    x[5, 256:384] = np.arange(128, dtype=np.uint16)              # bf16 subnormals
    x[6, 384:512] = (np.arange(128, dtype=np.uint16) | 0x8000)   # negative subnormals
    x[7, :128] = synth.bf16_bits_from_f32(np.full(128, 3.0e38, np.float32))   # near bf16 max
    x[8, :128] = synth.bf16_bits_from_f32(np.linspace(-1e-30, 1e-30, 128).astype(np.float32))
    x[9, :128] = 1                                               # the smallest subnormal everywhere
    _assert_rowgroup(x, "edge groups", mode=FP32)
    for rows in (1, 3, 17, 257):
        _assert_rowgroup(synth.normal_bf16((rows, 384), 1.0, 40, rows), f"ragged rows={rows}", mode=FP32)


def test_fp32_scale_division_sweep_all_orientations():
    x = _division_sweep()
    _assert_rowgroup(x, "division sweep", mode=FP32)
    _assert_dual(x, "division sweep, row side", mode=FP32)
    xt = np.ascontiguousarray(x.T)
    _assert_dual(xt, "division sweep, column side", mode=FP32)
    _assert_colgroup(xt[:, :4096], "division sweep, colgroup", mode=FP32)


def test_fp32_scale_decoder_layer_dual_and_colgroup():
    for lin in synth.decoder_layer():
        _assert_dual(lin["x"], f"X {lin['name']}", mode=FP32)
        _assert_dual(lin["dy"], f"dY {lin['name']}", mode=FP32)
    lin = synth.decoder_layer()[0]
    _assert_colgroup(lin["x"], "X qkv", mode=FP32)


def test_fp32_scale_outlier_stress_and_strided():
    x, _, _ = synth.outlier_stress()
    _assert_rowgroup(x, "outlier X", mode=FP32)
    _assert_dual(x, "outlier X", mode=FP32)
    wide = synth.normal_bf16((1024, 4096), 1.0, 48, 0)
    _assert_dual(wide, "column slice, padded outputs", cols=2048, pad_q=256, pad_qT=128, mode=FP32)


def test_fp32_scale_block():
    w = synth.normal_bf16((384, 256), 0.02, 45, 0)
    w[128:256, 128:256] = 0
    w[:128, :128] = np.arange(128 * 128, dtype=np.uint16).reshape(128, 128) % 128   # subnormal block
    _assert_block(w, "edges", mode=FP32)
    _assert_block(w, "edges, no transpose", transpose=False, mode=FP32)
    _, w = synth.single_linear()
    _assert_block(w, "12288x2048 W", mode=FP32)



def test_fp32_scale_quotient_exhaustive():
    """Under the amax/448 rule the quantizers form x/s from a reciprocal and
    one fused-multiply-add correction.  The probe compares that with a plain
    IEEE division for every non-negative finite bf16 amax and every bf16 x
    with |x| <= amax, both signs (about 10^9 elements, every element a
    quantizer can see): the stored scale and the E4M3 code must agree.  The
    oracle divides; the tests above tie the quantizers to it on their inputs,
    and this check extends the agreement to all inputs."""
    import ctypes
    import os
    import torch
    import blockwise_fp8_linear_amd as fb
    note("fp8probe_fp32_quotient_check: grid 128 x 32640")
    lib = ctypes.CDLL(os.path.join(os.path.dirname(fb.LIB_PATH), "libfp8probe.so"))
    lib.fp8probe_fp32_quotient_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.fp8probe_fp32_quotient_check.restype = ctypes.c_int
    counts = torch.full((128 * 0x7F80,), -1, dtype=torch.int32, device="cuda")
    assert lib.fp8probe_fp32_quotient_check(counts.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    c = host(counts)
    assert c.min() >= 0, "the probe left blocks unwritten"
    bad = np.flatnonzero(c)
    assert bad.size == 0, f"{int(c.sum())} elements differ; first at amax bits {hex(int(bad[0]) // 128)}"


def test_pow2_scaled_conversion_exhaustive():
    """The power-of-two quantizers convert with the scaled instruction given
    the stored scale: for every bf16 pattern and every scale exponent the
    rule produces, wherever the quotient is in range, it must give the code
    of the exact quotient (the fp32 path: exact product, then the plain
    conversion, which the cast tests tie to the oracle)."""
    import ctypes
    import os
    import torch
    import blockwise_fp8_linear_amd as fb
    note("fp8probe_pow2_cvt_check: grid 256 x 253")
    lib = ctypes.CDLL(os.path.join(os.path.dirname(fb.LIB_PATH), "libfp8probe.so"))
    lib.fp8probe_pow2_cvt_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.fp8probe_pow2_cvt_check.restype = ctypes.c_int
    counts = torch.full((256 * 253,), -1, dtype=torch.int32, device="cuda")
    assert lib.fp8probe_pow2_cvt_check(counts.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    c = host(counts)
    assert c.min() >= 0, "the probe left blocks unwritten"
    bad = np.flatnonzero(c)
    assert bad.size == 0, f"{int(c.sum())} conversions differ; first at e = {int(bad[0]) // 256 - 126}"


def _sweep_values():
    """Every non-negative finite bf16 magnitude up to 448 and its negative."""
    mags = (np.arange(0x8000, dtype=np.uint32) << 16).view(np.float32)
    mags = mags[np.isfinite(mags) & (mags <= 448.0)]
    return np.concatenate([mags, -mags]).astype(np.float32)


def test_colgroup_exhaustive_cast():
    """The row-group kernel's exhaustive cast sweep through the separate
    column-group kernel: each column a group of 128 rows whose amax is
    exactly 448 * 2^e (row 0), the other 127 rows every bf16 magnitude up to
    448 scaled by 2^e, for every e in [-126, 118]."""
    vals = _sweep_values()
    per = 127
    ng = (vals.size + per - 1) // per
    vals = np.concatenate([vals, np.zeros(ng * per - vals.size, np.float32)]).reshape(ng, per)
    cols = []
    for e in range(-126, 119):
        blk = np.empty((ng, 128), np.float32)
        blk[:, 0] = 448.0 * np.float32(2.0 ** e)
        blk[:, 1:] = vals * np.float32(2.0 ** e)
        cols.append(blk)
    x = np.concatenate(cols)                                    # groups as rows
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 128, 128), np.float32)])
    _assert_colgroup(np.ascontiguousarray(synth.bf16_bits_from_f32(x).T), "exhaustive cast")


def test_block_exhaustive_cast():
    """The same sweep through the block quantizer (and its transposed copy):
    each 128 x 128 block holds amax 448 * 2^e at (0, 0) and 16383 of the
    scaled magnitudes, every magnitude appearing at every e in [-126, 118]."""
    vals = _sweep_values()
    per = 128 * 128 - 1
    nb = (vals.size + per - 1) // per
    vals = np.concatenate([vals, np.zeros(nb * per - vals.size, np.float32)]).reshape(nb, per)
    blocks = []
    for e in range(-126, 119):
        b = np.empty((nb, 128 * 128), np.float32)
        b[:, 0] = 448.0 * np.float32(2.0 ** e)
        b[:, 1:] = vals * np.float32(2.0 ** e)
        blocks.append(b.reshape(nb, 128, 128))
    w = np.concatenate(blocks)                                  # [blocks, 128, 128]
    w = np.ascontiguousarray(w.transpose(1, 0, 2).reshape(128, -1))   # blocks side by side
    _assert_block(synth.bf16_bits_from_f32(w), "exhaustive cast")
