"""GPU parity of the block-scaled Fprop / Dgrad / Wgrad GEMMs against the CPU
oracle, through the C ABI, for both accumulation algorithms.

Tolerance -- the reading of "within max relative error 1e-3 of the oracle's
fp32-accumulated result computed from the same quantized operands":
  * fp32 output: per element |y - y32| <= 1e-3 * D, with D the sum of the
    absolute values of all scaled products (the quantity any summation-order
    error is proportional to), and normwise max|y - y32| <= 1e-3 * max|y32|.
    An elementwise |y - y32| / |y32| bound cannot hold for any summation order
    near cancellation, so it is not gated.
  * bf16 output: bit-equal to the round-to-nearest-even of the same kernel's
    fp32 result, and within half a bf16 ulp (<= 2^-8 |y32|) plus the fp32
    gate above of the oracle's result.
Exact cases: integer-valued operands in [-16, 16] quantize losslessly and
every partial sum is an integer below 2^24, so the GPU result must equal an
int64 matmul exactly (and its bf16 rounding, bit for bit).

The GPU path quantizes its own operands; the oracle quantizes the same seeded
bf16 inputs on the host (the quantizers are checked bit-exact separately).
"""
import numpy as np
import pytest

import oracle
import blockwise_fp8_linear_amd as fb
from blockwise_fp8_linear_amd import synth
from gpu_util import check_bf16, check_f32, dev_bf16, host, host_f32, note, require_gpu, sample_rows

pytestmark = pytest.mark.gpu

ALGOS = {"promote": fb.FP8BLK_ALGO_PROMOTE, "scaled": fb.FP8BLK_ALGO_SCALED_MFMA}
OPS = ("fprop", "dgrad", "wgrad")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def varied(shape, std, key):
    """N(0, std^2) with each 128x128 block scaled by its own power of two, so
    that row-group, column-group and block scales all vary."""
    rng = synth.rng_for(*key)
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    R, C = shape
    f = 2.0 ** rng.integers(-5, 6, size=((R + 127) // 128, (C + 127) // 128))
    x *= np.repeat(np.repeat(f, 128, 0)[:R], 128, 1)[:, :C].astype(np.float32)
    return synth.bf16_bits_from_f32(x)


class Layer:
    """One linear's operands, quantized on the GPU and by the oracle, under
    scale rule `mode` (0 power of two, 1 amax / 448)."""

    def __init__(self, x, w, dy, mode=0):
        import torch
        self.M, self.K = x.shape
        self.N = w.shape[0]
        self.mode = mode
        xt, wt, dyt = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
        self.g = {}
        self.g["qx"], self.g["sx"] = fb.fp8_quantize_rowgroup(xt, scale_mode=mode)
        self.g["qxT"], self.g["sxT"] = fb.fp8_quantize_colgroup(xt, scale_mode=mode)
        self.g["qw"], self.g["qwT"], self.g["sw"] = fb.fp8_quantize_block(wt, scale_mode=mode)
        self.g["qdy"], self.g["sdy"] = fb.fp8_quantize_rowgroup(dyt, scale_mode=mode)
        self.g["qdyT"], self.g["sdyT"] = fb.fp8_quantize_colgroup(dyt, scale_mode=mode)
        torch.cuda.synchronize()
        self.o = {}
        self.o["qx"], self.o["sx"] = oracle.quantize_rowgroup(x, mode=mode)
        self.o["qxT"], self.o["sxT"] = oracle.quantize_colgroup(x, mode=mode)
        self.o["qw"], _, self.o["sw"] = oracle.quantize_block(w, transpose=False, mode=mode)
        self.o["qdy"], self.o["sdy"] = oracle.quantize_rowgroup(dy, mode=mode)
        self.o["qdyT"], self.o["sdyT"] = oracle.quantize_colgroup(dy, mode=mode)

    def gpu(self, op, algo, out_dtype, out=None):
        g = self.g
        args = {"fprop": (g["qx"], g["sx"], g["qw"], g["sw"]),
                "dgrad": (g["qdy"], g["sdy"], g["qwT"], g["sw"]),
                "dgrad_w": (g["qdy"], g["sdy"], g["qw"], g["sw"]),
                "wgrad": (g["qdyT"], g["sdyT"], g["qxT"], g["sxT"])}[op]
        opc = {"fprop": fb.FP8BLK_OP_FPROP, "dgrad": fb.FP8BLK_OP_DGRAD, "dgrad_w": fb.FP8BLK_OP_DGRAD_W,
               "wgrad": fb.FP8BLK_OP_WGRAD}[op]
        return fb.fp8_block_gemm(opc, *args, self.M, self.N, self.K, out_dtype=out_dtype, algo=algo, out=out,
                                 scale_mode=self.mode)

    def ref(self, op, rows):
        o = self.o
        if op == "fprop":
            return oracle.gemm_fprop(o["qx"], o["sx"], o["qw"], o["sw"], rows=rows)
        if op in ("dgrad", "dgrad_w"):
            return oracle.gemm_dgrad(o["qdy"], o["sdy"], o["qw"], o["sw"], rows=rows)
        return oracle.gemm_wgrad(o["qdyT"], o["sdyT"], o["qxT"], o["sxT"], rows=rows)

    def out_rows(self, op):
        return self.N if op == "wgrad" else self.M

    def out_shape(self, op):
        return {"fprop": (self.M, self.N), "wgrad": (self.N, self.K)}.get(op, (self.M, self.K))


def nan_filled(shape, dtype):
    """An output buffer holding NaN everywhere (bf16 0xFFFF, fp32 0xFFFFFFFF),
    so that any element a kernel fails to write shows up as non-finite."""
    import torch
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xFF)
    return t


def check_op(layer, op, algo_name, rows=None, what=""):
    import torch
    algo = ALGOS[algo_name]
    nrows = layer.out_rows(op)
    rows = np.arange(nrows) if rows is None else np.asarray(rows)
    y32, _, bound = layer.ref(op, rows)
    # NaN-filled outputs: every element of both must be written (finite),
    # including the rows the oracle does not recompute
    yf = layer.gpu(op, algo, torch.float32, out=nan_filled(layer.out_shape(op), torch.float32))
    yb = layer.gpu(op, algo, torch.bfloat16, out=nan_filled(layer.out_shape(op), torch.bfloat16))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(yf).all()) and bool(torch.isfinite(yb).all()), f"{op} {algo_name}: unwritten outputs"

    yf_h = host_f32(yf)[rows]
    yb_h = host(yb)[rows]
    tag = f"{what} {op} {algo_name} M={layer.M} N={layer.N} K={layer.K}"
    stats = check_f32(yf_h, y32, bound, tag)
    check_bf16(yb_h, yf_h, y32, bound, tag)
    note(f"{tag}: err/bound {stats['err/bound']:.2e} normwise {stats['normwise']:.2e} "
         f"bit-exact-vs-oracle-fp32 {stats['exact_frac']:.3f}")
    return stats


@pytest.mark.parametrize("algo", list(ALGOS))
# (M, N, K): ragged edges against 256-wide tiles; reductions whose block count
# is / is not a multiple of 4 (the 256x256 block-scaled-MFMA kernel takes the
# former, the general kernel the latter)
@pytest.mark.parametrize("shape", [(384, 640, 512), (640, 384, 1024), (1024, 512, 384), (256, 128, 640),
                                   (128, 384, 256), (640, 256, 1152)])
def test_small_shapes_all_ops(algo, shape):
    M, N, K = shape
    key = (60, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)))
    for op in OPS:
        check_op(layer, op, algo, what="small")


@pytest.mark.parametrize("algo", list(ALGOS))
def test_exact_integer_products(algo):
    import torch
    M, N, K = 256, 384, 640
    x = synth.integer_valued_bf16((M, K), -16, 16, 61, 0)
    w = synth.integer_valued_bf16((N, K), -16, 16, 61, 1)
    dy = synth.integer_valued_bf16((M, N), -16, 16, 61, 2)
    layer = Layer(x, w, dy)
    X, W, DY = (oracle.bf16_to_f64(a).astype(np.int64) for a in (x, w, dy))
    exact = {"fprop": X @ W.T, "dgrad": DY @ W, "wgrad": DY.T @ X}
    for op in OPS:
        yf = host_f32(layer.gpu(op, ALGOS[algo], torch.float32))
        yb = host(layer.gpu(op, ALGOS[algo], torch.bfloat16))
        assert np.array_equal(yf.astype(np.int64), exact[op]), f"{op} {algo}: not exact"
        assert np.array_equal(yf, exact[op].astype(np.float32))
        rne = oracle.bf16_rne(exact[op].astype(np.float32))
        assert np.array_equal(yb, rne), f"{op} {algo}: bf16 rounding of the exact result differs"


def test_tiny_fprop_config():
    """The 256x256 fprop workload, every output element."""
    import torch
    x, w = synth.tiny_fprop()
    layer = Layer(x, w, synth.normal_bf16((256, 256), 1e-3, 0, 1, 2))
    for algo in ALGOS:
        check_op(layer, "fprop", algo, what="tiny")


def _sample_rows(n, key, k=24):
    """Output rows for the oracle to recompute: the edges, k random rows, and
    one random row in every 256-row band, so that every output tile (and, in
    the stream-K kernels, every shared tile and its fix-up) is compared; each
    row is compared over all its columns."""
    return sample_rows(n, synth.rng_for(*key), k)


def test_single_linear_fprop_full_size():
    """8192 x 12288 x 2048 fprop in the benchmark's launch configuration, on
    sampled output rows (every column of each)."""
    import torch
    x, w = synth.single_linear()
    xt, wt = dev_bf16(x), dev_bf16(w)
    qx, sx = fb.fp8_quantize_rowgroup(xt)
    qw, _, sw = fb.fp8_quantize_block(wt, transpose=False)
    ox, osx = oracle.quantize_rowgroup(x)
    ow, _, osw = oracle.quantize_block(w, transpose=False)
    rows = _sample_rows(8192, (62, 0))
    y32, _, bound = oracle.gemm_fprop(ox, osx, ow, osw, rows=rows)
    for algo_name, algo in ALGOS.items():
        yf = fb.fp8_block_gemm(fb.FP8BLK_OP_FPROP, qx, sx, qw, sw, 8192, 12288, 2048, out_dtype=torch.float32, algo=algo,
                               out=nan_filled((8192, 12288), torch.float32))
        yb = fb.fp8_block_gemm(fb.FP8BLK_OP_FPROP, qx, sx, qw, sw, 8192, 12288, 2048, algo=algo,
                               out=nan_filled((8192, 12288), torch.bfloat16))
        torch.cuda.synchronize()
        assert bool(torch.isfinite(yf).all()) and bool(torch.isfinite(yb).all()), "unwritten outputs"
        yf_h, yb_h = host_f32(yf)[rows], host(yb)[rows]
        st = check_f32(yf_h, y32, bound, f"single linear {algo_name}")
        check_bf16(yb_h, yf_h, y32, bound, f"single linear {algo_name}")
        note(f"single linear fprop {algo_name}: {st}")


def test_outlier_stress_fprop_full_size():
    import torch
    x, w, _ = synth.outlier_stress()
    xt, wt = dev_bf16(x), dev_bf16(w)
    qx, sx = fb.fp8_quantize_rowgroup(xt)
    qw, _, sw = fb.fp8_quantize_block(wt, transpose=False)
    ox, osx = oracle.quantize_rowgroup(x)
    ow, _, osw = oracle.quantize_block(w, transpose=False)
    rows = _sample_rows(8192, (63, 0))
    y32, _, bound = oracle.gemm_fprop(ox, osx, ow, osw, rows=rows)
    for algo_name, algo in ALGOS.items():
        yf = fb.fp8_block_gemm(fb.FP8BLK_OP_FPROP, qx, sx, qw, sw, 8192, 12288, 2048, out_dtype=torch.float32, algo=algo,
                               out=nan_filled((8192, 12288), torch.float32))
        yb = fb.fp8_block_gemm(fb.FP8BLK_OP_FPROP, qx, sx, qw, sw, 8192, 12288, 2048, algo=algo,
                               out=nan_filled((8192, 12288), torch.bfloat16))
        torch.cuda.synchronize()
        assert bool(torch.isfinite(yf).all()) and bool(torch.isfinite(yb).all()), "unwritten outputs"
        yf_h, yb_h = host_f32(yf)[rows], host(yb)[rows]
        st = check_f32(yf_h, y32, bound, f"outlier {algo_name}")
        check_bf16(yb_h, yf_h, y32, bound, f"outlier {algo_name}")
        note(f"outlier fprop {algo_name}: {st}")


@pytest.mark.parametrize("li", range(4))
def test_decoder_layer_full_size(li):
    """Each linear of the decoder layer at 8192 tokens: fprop, dgrad and wgrad
    on sampled output rows, both algorithms."""
    lin = synth.decoder_layer(linears=(synth.LAYER_LINEARS[li],))[0]
    layer = Layer(lin["x"], lin["w"], lin["dy"])
    for op in OPS:
        rows = _sample_rows(layer.out_rows(op), (64, li, OPS.index(op)), k=8)
        for algo in ALGOS:
            check_op(layer, op, algo, rows=rows, what=f"layer {lin['name']}")


# ---- scales by the amax / 448 rule (FP8BLK_SCALE_FP32): not powers of two,
# so only the promote algorithm takes them; the same tolerance bar.

@pytest.mark.parametrize("shape", [(384, 640, 512), (640, 384, 1024), (1024, 512, 384), (256, 128, 640),
                                   (640, 256, 1152)])
def test_fp32_scales_promote_small_shapes(shape):
    M, N, K = shape
    key = (66, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)), mode=1)
    assert not np.all(np.frexp(oracle.quantize_rowgroup(varied((M, K), 1.0, key + (0,)), mode=1)[1])[0] == 0.5)
    for op in OPS:
        check_op(layer, op, "promote", what="fp32 scales")


@pytest.mark.parametrize("li", [0, 3])
def test_fp32_scales_promote_decoder_layer_full_size(li):
    """QKV and down-projection linears at 8192 tokens with amax / 448 scales:
    fprop, dgrad and wgrad (stream-K) on sampled output rows."""
    lin = synth.decoder_layer(linears=(synth.LAYER_LINEARS[li],))[0]
    layer = Layer(lin["x"], lin["w"], lin["dy"], mode=1)
    for op in OPS:
        rows = _sample_rows(layer.out_rows(op), (67, li, OPS.index(op)), k=8)
        check_op(layer, op, "promote", rows=rows, what=f"fp32 scales, layer {lin['name']}")


def test_named_entry_points_and_determinism():
    """The named C entry points (default algorithm) equal the generic one, and
    repeated runs -- including the stream-K Wgrad -- are bit-identical."""
    import torch
    M, N, K = 8192, 2048, 256
    layer = Layer(synth.normal_bf16((M, K), 1.0, 65, 0), synth.normal_bf16((N, K), 0.02, 65, 1),
                  synth.normal_bf16((M, N), 1e-3, 65, 2))
    g = layer.g
    assert fb.fp8_block_gemm_workspace_size(fb.FP8BLK_OP_WGRAD, M, N, K) > 0
    a = fb.fp8_block_gemm_wgrad(g["qdyT"], g["sdyT"], g["qxT"], g["sxT"])
    b = fb.fp8_block_gemm_wgrad(g["qdyT"], g["sdyT"], g["qxT"], g["sxT"])
    c = layer.gpu("wgrad", fb.FP8BLK_ALGO_DEFAULT, torch.bfloat16)
    f1 = fb.fp8_block_gemm_fprop(g["qx"], g["sx"], g["qw"], g["sw"])
    f2 = layer.gpu("fprop", fb.FP8BLK_ALGO_DEFAULT, torch.bfloat16)
    d1 = fb.fp8_block_gemm_dgrad(g["qdy"], g["sdy"], g["qwT"], g["sw"])
    d2 = layer.gpu("dgrad", fb.FP8BLK_ALGO_DEFAULT, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
    assert torch.equal(f1, f2) and torch.equal(d1, d2)
    rows = _sample_rows(N, (65, 3), k=8)
    check_op(layer, "wgrad", "promote", rows=rows, what="stream-K")
    check_op(layer, "wgrad", "scaled", rows=rows, what="stream-K")


# Wgrad shapes (M, N, K) that exercise the persistent Wgrad kernel of the
# 256x256 path (a data-parallel wave of whole tiles, then stream-K over the
# rest): one output tile shared by 4 workgroups; 15 tiles with a ragged edge
# shared by up to 18 workgroups of 1-2 reduction units each (some pieces
# being a workgroup's last segment); 256 whole tiles, then 128 tiles split
# in two; one unit per tile (several whole tiles per workgroup, no
# workspace); 256 whole tiles, then 16 tiles in 4 pieces on 64 of the 256
# workgroups.
@pytest.mark.parametrize("shape", [(2048, 256, 256), (9216, 1152, 768), (1024, 4096, 6144), (512, 5120, 7680),
                                   (2048, 4352, 4096)])
def test_wgrad_streamk_partitions(shape):
    import torch
    M, N, K = shape
    key = (66, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)))
    rows = _sample_rows(N, key, k=16)
    check_op(layer, "wgrad", "scaled", rows=rows, what="stream-K")
    a = layer.gpu("wgrad", fb.FP8BLK_ALGO_SCALED_MFMA, torch.float32)
    b = layer.gpu("wgrad", fb.FP8BLK_ALGO_SCALED_MFMA, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "stream-K Wgrad is not deterministic"


# More output tiles than fit in one wave of workgroups, with ragged edges in
# both output dimensions: Fprop and Dgrad on 17 x 17 = 289 tiles; Wgrad on
# 17 x 16 tiles = one data-parallel wave plus stream-K over a ragged tile
# row.
@pytest.mark.parametrize("shape,ops", [((4224, 4224, 1024), ("fprop",)), ((4224, 1024, 4224), ("dgrad", "dgrad_w")),
                                       ((2048, 4224, 4096), ("wgrad",))])
def test_many_tiles_ragged(shape, ops):
    M, N, K = shape
    key = (67, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)))
    for op in ops:
        n = layer.out_rows(op)
        rows = np.unique(np.concatenate([_sample_rows(n, key + (len(op),), k=12),
                                         np.arange(n - 140, n)]))   # the whole ragged last tile row
        check_op(layer, op, "scaled", rows=rows, what="many tiles")


# fp32 accumulation into an existing output (FP8BLK_OUT_FP32_ACCUM, the fp32
# main-gradient case): the result must be exactly fl32(old + r), r being what
# FP8BLK_OUT_FP32 stores, for every op, both algorithms, and the Wgrad paths
# that sum partial tiles (the stream-K fix-ups of both GEMM paths).
@pytest.mark.parametrize("shape", [(1024, 4096, 6144), (2048, 256, 256), (640, 384, 1024), (4224, 4224, 512)])
def test_fp32_accumulate(shape):
    import torch
    M, N, K = shape
    key = (68, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)))
    g = layer.g
    args = {"fprop": (fb.FP8BLK_OP_FPROP, g["qx"], g["sx"], g["qw"], g["sw"], (M, N)),
            "dgrad": (fb.FP8BLK_OP_DGRAD, g["qdy"], g["sdy"], g["qwT"], g["sw"], (M, K)),
            "dgrad_w": (fb.FP8BLK_OP_DGRAD_W, g["qdy"], g["sdy"], g["qw"], g["sw"], (M, K)),
            "wgrad": (fb.FP8BLK_OP_WGRAD, g["qdyT"], g["sdyT"], g["qxT"], g["sxT"], (N, K))}
    gen = torch.Generator(device="cuda").manual_seed(68)
    for op, (opc, a, sa, b, sb, oshape) in args.items():
        for algo_name, algo in ALGOS.items():
            old = torch.randn(oshape, device="cuda", dtype=torch.float32, generator=gen)
            r = fb.fp8_block_gemm(opc, a, sa, b, sb, M, N, K, out_dtype=torch.float32, algo=algo)
            acc = old.clone()
            fb.fp8_block_gemm(opc, a, sa, b, sb, M, N, K, out_dtype=torch.float32, algo=algo, out=acc,
                              accumulate=True)
            torch.cuda.synchronize()
            want = host_f32(old) + host_f32(r)          # float32 + float32 in numpy: one rounding
            got = host_f32(acc)
            assert np.array_equal(got, want), f"{op} {algo_name} {shape}: accumulation differs"


def check_backward(layer, rows_dx, rows_dw, what):
    """fp8_block_gemm_backward (Dgrad and Wgrad in one call) against the
    oracle, fp32 and bf16 outputs, on the given output rows."""
    import torch
    g = layer.g
    args = (g["qdy"], g["sdy"], g["qwT"], g["sw"], g["qdyT"], g["sdyT"], g["qxT"], g["sxT"])
    M, N, K = layer.M, layer.N, layer.K
    dxf, dwf = fb.fp8_block_gemm_backward(*args, dx_dtype=torch.float32, dw_dtype=torch.float32,
                                          dx=nan_filled((M, K), torch.float32), dw=nan_filled((N, K), torch.float32),
                                          scale_mode=layer.mode)
    dxb, dwb = fb.fp8_block_gemm_backward(*args, dx=nan_filled((M, K), torch.bfloat16),
                                          dw=nan_filled((N, K), torch.bfloat16), scale_mode=layer.mode)
    torch.cuda.synchronize()
    for t in (dxf, dwf, dxb, dwb):
        assert bool(torch.isfinite(t).all()), f"{what}: unwritten backward outputs"
    for op, rows, yf, yb in (("dgrad", rows_dx, dxf, dxb), ("wgrad", rows_dw, dwf, dwb)):
        y32, _, bound = layer.ref(op, rows)
        tag = f"{what} backward/{op} M={layer.M} N={layer.N} K={layer.K}"
        st = check_f32(host_f32(yf)[rows], y32, bound, tag)
        check_bf16(host(yb)[rows], host_f32(yf)[rows], y32, bound, tag)
        note(f"{tag}: err/bound {st['err/bound']:.2e} normwise {st['normwise']:.2e}")
    return dxf, dwf


# (M, N, K): fused launches (M and N multiples of 512) with one, several or
# shared tiles and a ragged K edge; (384, 640, 512) takes the two-call path.
@pytest.mark.parametrize("shape", [(1024, 512, 384), (512, 1024, 640), (2048, 1536, 1152), (384, 640, 512)])
def test_backward_small(shape):
    import torch
    M, N, K = shape
    key = (69, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)))
    dxf, dwf = check_backward(layer, np.arange(M), np.arange(N), "small")
    # deterministic, and fp32 accumulation into dW
    g = layer.g
    args = (g["qdy"], g["sdy"], g["qwT"], g["sw"], g["qdyT"], g["sdyT"], g["qxT"], g["sxT"])
    dx2, dw2 = fb.fp8_block_gemm_backward(*args, dx_dtype=torch.float32, dw_dtype=torch.float32)
    old = torch.randn((N, K), device="cuda", dtype=torch.float32, generator=torch.Generator(device="cuda").manual_seed(69))
    acc = old.clone()
    fb.fp8_block_gemm_backward(*args, dx_dtype=torch.float32, dw_dtype=torch.float32, dw=acc, accumulate_dw=True)
    torch.cuda.synchronize()
    assert torch.equal(dxf, dx2) and torch.equal(dwf, dw2), "backward is not deterministic"
    assert np.array_equal(host_f32(acc), host_f32(old) + host_f32(dwf)), "dW accumulation differs"


@pytest.mark.parametrize("shape", [(1024, 512, 384), (384, 640, 512)])
def test_fp32_scales_route_to_promote(shape):
    """amax / 448 scales told to the GEMMs by scale_mode: DEFAULT runs the
    promote algorithm (bit-identical to asking for it), the block-scaled MFMA
    is refused before any launch, and the backward call runs both
    contractions with the promote algorithm, within the tolerance of the
    oracle's fp32-scale results."""
    import torch
    M, N, K = shape
    key = (72, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)), mode=1)
    for op in OPS:
        a = layer.gpu(op, fb.FP8BLK_ALGO_DEFAULT, torch.float32)
        b = layer.gpu(op, fb.FP8BLK_ALGO_PROMOTE, torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"{op}: DEFAULT with fp32 scales is not PROMOTE"
        with pytest.raises(RuntimeError, match="bad enum"):
            layer.gpu(op, fb.FP8BLK_ALGO_SCALED_MFMA, torch.float32)
    dxf, dwf = check_backward(layer, np.arange(M), np.arange(N), "fp32 scales")
    dx = layer.gpu("dgrad", fb.FP8BLK_ALGO_PROMOTE, torch.float32)
    dw = layer.gpu("wgrad", fb.FP8BLK_ALGO_PROMOTE, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(dxf, dx) and torch.equal(dwf, dw), "backward with fp32 scales is not the promote pair"


@pytest.mark.parametrize("li", range(4))
def test_backward_decoder_layer_full_size(li):
    """The fused backward of each decoder-layer linear at 8192 tokens (the
    benchmark's launch), sampled output rows of dX and dW."""
    lin = synth.decoder_layer(linears=(synth.LAYER_LINEARS[li],))[0]
    layer = Layer(lin["x"], lin["w"], lin["dy"])
    check_backward(layer, _sample_rows(layer.M, (71, li, 0), k=8), _sample_rows(layer.N, (71, li, 1), k=8),
                   f"layer {lin['name']}")


# ---- Dgrad from the weight codes as quantized (fp8_block_gemm_dgrad_w,
# FP8BLK_OP_DGRAD_W): the oracle's Dgrad reads W[n][k] directly; the kernels
# stage [n][k] tiles and form fragments with LDS transpose reads.  Each lane
# then holds the same bytes in the same reduction order as with the
# transposed copy, so the result must also equal the qwT path bit for bit.

def check_dgrad_w(layer, algo_name, rows=None, what=""):
    import torch
    stats = check_op(layer, "dgrad_w", algo_name, rows=rows, what=what)
    for dt in (torch.float32, torch.bfloat16):
        a = layer.gpu("dgrad_w", ALGOS[algo_name], dt)
        b = layer.gpu("dgrad", ALGOS[algo_name], dt)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"{what} {algo_name} {dt}: dgrad from qw differs from dgrad from qwT"
    return stats


@pytest.mark.parametrize("algo", list(ALGOS))
# reductions N with 128-block counts that are / are not multiples of 4 (the
# fast kernel / the general one), ragged M, and output widths K that end
# half-way through a 256-wide tile (the clamped column chunks)
@pytest.mark.parametrize("shape", [(384, 640, 512), (640, 512, 384), (1024, 384, 640), (256, 1152, 128),
                                   (640, 1024, 1152), (128, 512, 896)])
def test_dgrad_w_small_shapes(algo, shape):
    M, N, K = shape
    key = (68, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)))
    check_dgrad_w(layer, algo, what="dgrad_w small")


@pytest.mark.parametrize("li", range(4))
def test_dgrad_w_and_backward_w_decoder_layer_full_size(li):
    """Each linear of the decoder layer at 8192 tokens: Dgrad from qw against
    the oracle on sampled rows and against the qwT path bit for bit; the
    fused backward from qw against the fused backward from qwT, both
    outputs bit for bit."""
    import torch
    lin = synth.decoder_layer(linears=(synth.LAYER_LINEARS[li],))[0]
    layer = Layer(lin["x"], lin["w"], lin["dy"])
    rows = _sample_rows(layer.M, (69, li), k=8)
    check_dgrad_w(layer, "scaled", rows=rows, what=f"layer {lin['name']}")
    g = layer.g
    for dxt in (torch.bfloat16, torch.float32):
        a = fb.fp8_block_gemm_backward_w(g["qdy"], g["sdy"], g["qw"], g["sw"], g["qdyT"], g["sdyT"], g["qxT"],
                                         g["sxT"], dx_dtype=dxt)
        b = fb.fp8_block_gemm_backward(g["qdy"], g["sdy"], g["qwT"], g["sw"], g["qdyT"], g["sdyT"], g["qxT"],
                                       g["sxT"], dx_dtype=dxt)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), f"backward_w {lin['name']} {dxt}"


@pytest.mark.parametrize("shape", [(1024, 512, 384), (512, 1024, 640), (384, 640, 512)])
def test_backward_w_small(shape):
    """The fused backward from qw (and its two-call fallback shapes) against
    the oracle for both outputs."""
    import torch
    M, N, K = shape
    key = (70, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)))
    g = layer.g
    dx, dw = fb.fp8_block_gemm_backward_w(g["qdy"], g["sdy"], g["qw"], g["sw"], g["qdyT"], g["sdyT"], g["qxT"],
                                          g["sxT"], dx_dtype=torch.float32, dw_dtype=torch.float32)
    torch.cuda.synchronize()
    for out, op in ((dx, "dgrad"), (dw, "wgrad")):
        y32, _, bound = layer.ref(op, np.arange(layer.out_rows(op)))
        check_f32(host_f32(out), y32, bound, f"backward_w {op} {shape}")


def test_dgrad_w_fp32_scales_promote():
    """amax / 448 scales: the promote kernel's transposed-B configuration."""
    M, N, K = 640, 1024, 384
    key = (71, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)), mode=1)
    check_dgrad_w(layer, "promote", what="dgrad_w fp32 scales")



# ---- a seeded sweep of shapes through the default path: every contraction
# (Dgrad in both forms, the fused backward from the weight codes) against the
# oracle on sampled rows.  Ragged tile edges, reductions whose 128-block count
# is or is not a multiple of 4, and more tiles than CUs all come up.

def _sweep_shapes(n=16):
    rng = synth.rng_for(72, 0)
    return [tuple(int(v) * 128 for v in rng.integers(1, (33, 25, 25))) for _ in range(n)]


@pytest.mark.parametrize("shape", _sweep_shapes())
def test_shape_sweep_default_path(shape):
    import torch
    M, N, K = shape
    key = (73, M, N, K)
    layer = Layer(varied((M, K), 1.0, key + (0,)), varied((N, K), 0.02, key + (1,)),
                  varied((M, N), 1e-3, key + (2,)))
    for op in ("fprop", "dgrad", "wgrad"):
        rows = _sample_rows(layer.out_rows(op), key + (len(op),), k=6)
        check_op(layer, op, "scaled", rows=rows, what="sweep")
    check_dgrad_w(layer, "scaled", rows=_sample_rows(M, key + (9,), k=6), what="sweep")
    g = layer.g
    dx, dw = fb.fp8_block_gemm_backward_w(g["qdy"], g["sdy"], g["qw"], g["sw"], g["qdyT"], g["sdyT"], g["qxT"],
                                          g["sxT"], dx_dtype=torch.float32, dw_dtype=torch.float32)
    torch.cuda.synchronize()
    for out, op in ((dx, "dgrad"), (dw, "wgrad")):
        rows = _sample_rows(layer.out_rows(op), key + (10 + len(op),), k=6)
        y32, _, bound = layer.ref(op, rows)
        check_f32(host_f32(out)[rows], y32, bound, f"sweep backward_w {op} {shape}")


# ---- the longest reduction the 256x256 kernel takes with weight-block
# scales (128 blocks, every scale of the tile's block column held in LDS) and
# the next length up (132 blocks: the general kernel, and the fused backward
# falls back to two calls).

@pytest.mark.parametrize("R", [128 * 128, 132 * 128])
def test_weight_block_reduction_limit(R):
    import torch
    key = (74, R)
    rows = _sample_rows(512, key + (0,), k=8)
    # Fprop with K = R
    fwd = Layer(varied((512, R), 1.0, key + (1,)), varied((384, R), 0.02, key + (2,)),
                varied((512, 384), 1e-3, key + (3,)))
    check_op(fwd, "fprop", "scaled", rows=rows, what="limit")
    # Dgrad with N = R, both forms, and the backward from the weight codes
    bwd = Layer(varied((512, 384), 1.0, key + (4,)), varied((R, 384), 0.02, key + (5,)),
                varied((512, R), 1e-3, key + (6,)))
    check_op(bwd, "dgrad", "scaled", rows=rows, what="limit")
    check_dgrad_w(bwd, "scaled", rows=rows, what="limit")
    g = bwd.g
    dx, dw = fb.fp8_block_gemm_backward_w(g["qdy"], g["sdy"], g["qw"], g["sw"], g["qdyT"], g["sdyT"], g["qxT"],
                                          g["sxT"], dx_dtype=torch.float32, dw_dtype=torch.float32)
    torch.cuda.synchronize()
    for out, op, rr in ((dx, "dgrad", rows), (dw, "wgrad", _sample_rows(R, key + (7,), k=8))):
        y32, _, bound = bwd.ref(op, rr)
        check_f32(host_f32(out)[rr], y32, bound, f"limit backward_w {op} R={R}")
