"""The library's launches under HIP graph capture (through the C ABI, via the
binding): every call only enqueues work on the stream it is given -- here
torch's capture stream -- and needs no allocation, synchronisation or memset,
so a whole linear's step can be captured once and replayed.  Each replay
must reproduce the eager results bit for bit; the outputs are overwritten
with a fill and other eager work runs between replays."""
import numpy as np
import pytest

import blockwise_fp8_linear_amd as fb
from blockwise_fp8_linear_amd import synth
from gpu_util import dev_bf16, require_gpu

pytestmark = pytest.mark.gpu

M, N, K = 1024, 1536, 1024  # the fused backward and Wgrad both share tiles here (fix-up kernels run)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_linear_step_graph_replays_match_eager():
    import torch
    x = dev_bf16(synth.normal_bf16((M, K), 1.0, 80, 0))
    w = dev_bf16(synth.normal_bf16((N, K), 0.02, 80, 1))
    dy = dev_bf16(synth.normal_bf16((M, N), 1e-3, 80, 2))
    u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    o = {"qx": e((M, K), u8), "sx": e((M, K // 128), f32), "qxT": e((K, M), u8), "sxT": e((K, M // 128), f32),
         "qdy": e((M, N), u8), "sdy": e((M, N // 128), f32), "qdyT": e((N, M), u8), "sdyT": e((N, M // 128), f32),
         "qw": e((N, K), u8), "sw": e((N // 128, K // 128), f32),
         "y": e((M, N), bf16), "dx": e((M, K), bf16), "dw": e((N, K), f32), "dw2": e((N, K), bf16)}
    ws_b = e(fb.fp8_block_gemm_workspace_size(fb.FP8BLK_OP_BACKWARD, M, N, K), u8)
    ws_w = e(fb.fp8_block_gemm_workspace_size(fb.FP8BLK_OP_WGRAD, M, N, K), u8)
    assert ws_b.numel() > 0 and ws_w.numel() > 0

    def step():
        fb.fp8_quantize_block_batch([w], transpose=False, outs=[(o["qw"], None, o["sw"])])
        fb.fp8_quantize_dual(x, q=o["qx"], s=o["sx"], qT=o["qxT"], sT=o["sxT"])
        fb.fp8_block_gemm_fprop(o["qx"], o["sx"], o["qw"], o["sw"], out=o["y"])
        fb.fp8_quantize_dual(dy, q=o["qdy"], s=o["sdy"], qT=o["qdyT"], sT=o["sdyT"])
        fb.fp8_block_gemm_backward_w(o["qdy"], o["sdy"], o["qw"], o["sw"], o["qdyT"], o["sdyT"], o["qxT"], o["sxT"],
                                     dx=o["dx"], dw=o["dw"], dw_dtype=f32, workspace=ws_b)
        fb.fp8_block_gemm_wgrad(o["qdyT"], o["sdyT"], o["qxT"], o["sxT"], out=o["dw2"], workspace=ws_w)

    step()  # eager (also the first call on this device of every kernel)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in o.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    other = torch.randn(512, 512, device="cuda")
    for rep, fill in enumerate((0, 0x55, 0xFF)):
        for v in o.values():
            v.view(torch.uint8).fill_(fill)  # the replay must rewrite every output
        other = other @ other.T / 512.0         # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in o:
            assert torch.equal(o[k].view(torch.uint8), ref[k].view(torch.uint8)), f"replay {rep}: {k} differs"
    assert np.isfinite(other.cpu().numpy()).all()
