"""fp8_block_gemm_backward_w_noalloc, through the C ABI: the library's static
device scratch in place of a workspace.  Each call's outputs must equal those
of fp8_block_gemm_backward_w (which takes a workspace) bit for bit, and
agree with the oracle within the GEMM tolerance on sampled rows.  The calls
run back to back, each leaving its partial tiles in the shared scratch for
the next: a large shape, then a smaller one, then one whose partial tiles
take nearly all of the scratch; amax / 448 scales (the promote pair, whose
Wgrad's stream-K partial tiles go to the scratch); and a launch that would
need more than the scratch, refused before anything runs."""
import numpy as np
import pytest

import oracle
import blockwise_fp8_linear_amd as fb
from blockwise_fp8_linear_amd import synth
from gpu_util import check_bf16, check_f32, dev_bf16, host, host_f32, note, require_gpu, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _operands(M, N, K, key, mode):
    x = synth.normal_bf16((M, K), 1.0, *key, 0)
    w = synth.normal_bf16((N, K), 0.02, *key, 1)
    dy = synth.normal_bf16((M, N), 1e-3, *key, 2)
    qw, _, sw = fb.fp8_quantize_block(dev_bf16(w), transpose=False, scale_mode=mode)
    _, _, qxT, sxT = fb.fp8_quantize_dual(dev_bf16(x), scale_mode=mode)
    qdy, sdy, qdyT, sdyT = fb.fp8_quantize_dual(dev_bf16(dy), scale_mode=mode)
    return (qdy, sdy, qw, sw, qdyT, sdyT, qxT, sxT), (x, w, dy)


def _filled(shape, dtype):
    import torch
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xFF)  # NaN: every element must be written
    return t


def _one_call(M, N, K, key, mode=fb.FP8BLK_SCALE_POW2, oracle_rows=None):
    import torch
    ops, (x, w, dy) = _operands(M, N, K, key, mode)
    dx, dw = _filled((M, K), torch.bfloat16), _filled((N, K), torch.float32)
    fb.fp8_block_gemm_backward_w_noalloc(*ops, dx, dw, scale_mode=mode)
    rdx, rdw = fb.fp8_block_gemm_backward_w(*ops, dw_dtype=torch.float32, scale_mode=mode)
    # fp32 Dgrad from the same call form, for the bf16 rounding check
    dxf = fb.fp8_block_gemm_backward_w_noalloc(*ops, _filled((M, K), torch.float32), _filled((N, K), torch.float32),
                                               scale_mode=mode)[0]
    torch.cuda.synchronize()
    tag = f"noalloc {M}x{N}x{K} scale mode {mode}"
    assert torch.equal(dx, rdx), f"{tag}: dX differs from the workspace form"
    assert torch.equal(dw, rdw), f"{tag}: dW differs from the workspace form"
    if oracle_rows:
        rng = synth.rng_for(*key, 9)
        ow, _, osw = oracle.quantize_block(w, transpose=False, mode=mode)
        oxT, osxT = oracle.quantize_colgroup(x, mode=mode)
        ody, osdy = oracle.quantize_rowgroup(dy, mode=mode)
        odyT, osdyT = oracle.quantize_colgroup(dy, mode=mode)
        rows = sample_rows(M, rng, k=2)
        y32, _, bound = oracle.gemm_dgrad(ody, osdy, ow, osw, rows=rows)
        check_f32(host_f32(dxf)[rows], y32, bound, f"{tag} dgrad")
        check_bf16(host(dx)[rows], host_f32(dxf)[rows], y32, bound, f"{tag} dgrad")
        rows = sample_rows(N, rng, k=2)
        y32, _, bound = oracle.gemm_wgrad(odyT, osdyT, oxT, osxT, rows=rows)
        st = check_f32(host_f32(dw)[rows], y32, bound, f"{tag} wgrad")
        note(f"{tag}: wgrad err/bound {st['err/bound']:.2e}")


def test_noalloc_backward_calls_in_a_row():
    # O projection at 8192 tokens: 128 partial Wgrad tiles, 32 MiB of scratch
    _one_call(8192, 2048, 2048, (90, 0), oracle_rows=True)
    # a smaller input right after: 96 partial tiles over the previous contents
    _one_call(1024, 1536, 1024, (90, 1), oracle_rows=True)
    # 240 partial tiles: 60 of the 64 MiB
    _one_call(2048, 1536, 1152, (90, 2))
    # amax / 448 scales: Dgrad then Wgrad with the promote algorithm, the
    # Wgrad's 256 partial 256x128 tiles taking 32 MiB
    _one_call(8192, 2048, 2048, (90, 3), mode=fb.FP8BLK_SCALE_FP32, oracle_rows=True)
    _one_call(1024, 1536, 1024, (90, 4))


def test_noalloc_refuses_more_than_its_scratch():
    import torch
    M, N, K = 1536, 1536, 2560          # the fused launch: 288 partial 256x256 tiles, 72 MiB
    ops, _ = _operands(M, N, K, (91, 0), fb.FP8BLK_SCALE_POW2)
    dx, dw = _filled((M, K), torch.bfloat16), _filled((N, K), torch.bfloat16)
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError, match="scratch"):
        fb.fp8_block_gemm_backward_w_noalloc(*ops, dx, dw)
    torch.cuda.synchronize()
    assert bool((dx.view(torch.int16) == -1).all()) and bool((dw.view(torch.int16) == -1).all()), \
        "a refused call wrote its outputs"
    # the workspace form takes it; the down projection's shape fits the scratch
    rdx, rdw = fb.fp8_block_gemm_backward_w(*ops)
    M, N, K = 8192, 2048, 6144
    ops, _ = _operands(M, N, K, (91, 1), fb.FP8BLK_SCALE_POW2)
    dx, dw = _filled((M, K), torch.bfloat16), _filled((N, K), torch.bfloat16)
    fb.fp8_block_gemm_backward_w_noalloc(*ops, dx, dw)
    rdx, rdw = fb.fp8_block_gemm_backward_w(*ops)
    torch.cuda.synchronize()
    assert torch.equal(dx, rdx) and torch.equal(dw, rdw)
    assert np.isfinite(host_f32(dx)).all()
