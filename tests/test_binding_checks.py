"""The Python binding refuses operands whose shapes disagree with the extents
it passes to the C ABI (which cannot check them: it sees only pointers), so
that no kernel is launched to read or write past an allocation.

Runs on the CPU: the binding's device check is replaced by a dtype / rank
check, so that host tensors stand in for device ones, and the library is
replaced by a stub that fails the test if it is ever reached -- every case
below must be refused before any C call."""
import pytest
import torch

import blockwise_fp8_linear_amd as fb

u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16


@pytest.fixture(autouse=True)
def host_stand_ins(monkeypatch):
    def dev(t, dtype, name, ndim=2):
        if not isinstance(t, torch.Tensor):
            raise TypeError(name)
        if t.dtype != dtype:
            raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
        if t.dim() != ndim:
            raise ValueError(f"{name}: expected {ndim} dims")
        return t

    def no_library(*a, **k):
        pytest.fail("the C library was reached with mismatched operands")

    monkeypatch.setattr(fb, "_dev", dev)
    monkeypatch.setattr(fb, "load_library", no_library)


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


M, N, K = 256, 384, 512


def ops():
    """Correctly shaped operands of one linear (M tokens, N out, K in)."""
    return {"qx": z((M, K), u8), "sx": z((M, K // 128), f32), "qw": z((N, K), u8), "sw": z((N // 128, K // 128), f32),
            "qwT": z((K, N), u8), "qdy": z((M, N), u8), "sdy": z((M, N // 128), f32), "qdyT": z((N, M), u8),
            "sdyT": z((N, M // 128), f32), "qxT": z((K, M), u8), "sxT": z((K, M // 128), f32)}


def refused(fn, *args, match="expected shape", **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_fprop_shapes():
    o = ops()
    refused(fb.fp8_block_gemm_fprop, o["qx"], z((M, K // 128 - 1), f32), o["qw"], o["sw"])        # sx short
    refused(fb.fp8_block_gemm_fprop, o["qx"], o["sx"], z((N, K - 128), u8), o["sw"])              # K mismatch
    refused(fb.fp8_block_gemm_fprop, o["qx"], o["sx"], o["qw"], z((N // 128, K // 128 + 1), f32))  # sw
    refused(fb.fp8_block_gemm_fprop, o["qx"], o["sx"], o["qw"], o["sw"], out=z((M, N - 128), bf16))


def test_dgrad_shapes():
    o = ops()
    refused(fb.fp8_block_gemm_dgrad, o["qdy"], o["sdy"], z((K, N - 128), u8), o["sw"])
    refused(fb.fp8_block_gemm_dgrad, o["qdy"], z((M, 1), f32), o["qwT"], o["sw"])
    refused(fb.fp8_block_gemm_dgrad_w, o["qdy"], o["sdy"], z((N + 128, K), u8), o["sw"])
    refused(fb.fp8_block_gemm_dgrad_w, o["qdy"], o["sdy"], o["qw"], o["sw"], out=z((K, M), bf16).t(),
            match="contiguous")


def test_wgrad_shapes():
    o = ops()
    refused(fb.fp8_block_gemm_wgrad, o["qdyT"], o["sdyT"], z((K, M + 128), u8), o["sxT"])       # M mismatch
    refused(fb.fp8_block_gemm_wgrad, o["qdyT"], o["sdyT"], o["qxT"], z((K, M // 128 + 1), f32))
    refused(fb.fp8_block_gemm_wgrad, o["qdyT"], o["sdyT"], o["qxT"], o["sxT"], out=z((N, K + 128), f32),
            out_dtype=f32)


def test_generic_entry_checks_explicit_sizes():
    o = ops()
    # the tensors are those of (M, N, K) but the call claims a larger M
    refused(fb.fp8_block_gemm, fb.FP8BLK_OP_FPROP, o["qx"], o["sx"], o["qw"], o["sw"], 2 * M, N, K)
    refused(fb.fp8_block_gemm, fb.FP8BLK_OP_WGRAD, o["qdyT"], o["sdyT"], o["qxT"], o["sxT"], M, N, 2 * K)
    refused(fb.fp8_block_gemm, fb.FP8BLK_OP_DGRAD_W, o["qdy"], o["sdy"], o["qwT"], o["sw"], M, N, K)  # qwT for qw
    with pytest.raises(ValueError, match="not a contraction"):
        fb.fp8_block_gemm(fb.FP8BLK_OP_BACKWARD, o["qx"], o["sx"], o["qw"], o["sw"], M, N, K)


@pytest.mark.parametrize("fn,wkey", [(fb.fp8_block_gemm_backward, "qwT"), (fb.fp8_block_gemm_backward_w, "qw")])
def test_backward_shapes(fn, wkey):
    o = ops()
    base = [o["qdy"], o["sdy"], o[wkey], o["sw"], o["qdyT"], o["sdyT"], o["qxT"], o["sxT"]]
    for i, bad in ((4, z((N, M + 128), u8)), (5, z((N, 1), f32)), (6, z((K + 128, M), u8)), (7, z((K, 1), f32)),
                   (3, z((1, 1), f32))):
        args = list(base)
        args[i] = bad
        refused(fn, *args)
    refused(fn, *base, dx=z((M, K - 128), bf16))
    refused(fn, *base, dw=z((N, K), f32), dw_dtype=f32, dx=z((M, K + 128), bf16)[:, :K], match="contiguous")


def test_quantizer_output_shapes():
    x = z((M, K), bf16)
    refused(fb.fp8_quantize_rowgroup, x, q=z((M - 1, K), u8))
    refused(fb.fp8_quantize_rowgroup, x, s=z((M, K // 128 - 1), f32))
    refused(fb.fp8_quantize_colgroup, x, qT=z((K, M - 128), u8))
    refused(fb.fp8_quantize_colgroup, x, sT=z((K, 1), f32))
    refused(fb.fp8_quantize_dual, x, qT=z((K - 128, M), u8))
    refused(fb.fp8_quantize_dual, x, s=z((M, 1), f32))
    w = z((N, K), bf16)
    refused(fb.fp8_quantize_block, w, s=z((N // 128, 1), f32))
    refused(fb.fp8_quantize_block, w, qT=z((N, K), u8))
    refused(fb.fp8_quantize_block_batch, [w], outs=[(z((N, K), u8), None, z((1, 1), f32))])
    refused(fb.fp8_quantize_block_batch, [w], outs=[(z((N, K), u8), z((N, K), u8), z((N // 128, K // 128), f32))])
