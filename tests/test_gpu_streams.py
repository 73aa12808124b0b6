"""Two host threads driving the library on two streams at once (ctypes
releases the interpreter lock during the calls): the results equal those of
a single-stream run.  The library keeps no per-call state outside the
caller's buffers, so calls on different streams do not interfere."""
import threading

import pytest

import blockwise_fp8_linear_amd as fb
from blockwise_fp8_linear_amd import synth
from gpu_util import dev_bf16, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _linear(x, w, dy, stream):
    import torch
    qw, _, sw = fb.fp8_quantize_block(w, transpose=False, stream=stream)
    qx, sx, qxT, sxT = fb.fp8_quantize_dual(x, stream=stream)
    y = fb.fp8_block_gemm_fprop(qx, sx, qw, sw, stream=stream)
    qdy, sdy, qdyT, sdyT = fb.fp8_quantize_dual(dy, stream=stream)
    dx, dw = fb.fp8_block_gemm_backward_w(qdy, sdy, qw, sw, qdyT, sdyT, qxT, sxT, dw_dtype=torch.float32,
                                          stream=stream)
    return y, dx, dw


def test_two_threads_two_streams():
    import torch
    shapes = ((1024, 1536, 1024), (2048, 1024, 512))
    inputs = []
    for i, (M, N, K) in enumerate(shapes):
        inputs.append((dev_bf16(synth.normal_bf16((M, K), 1.0, 81, 3 * i)),
                       dev_bf16(synth.normal_bf16((N, K), 0.02, 81, 3 * i + 1)),
                       dev_bf16(synth.normal_bf16((M, N), 1e-3, 81, 3 * i + 2))))
    ref = [_linear(*inp, None) for inp in inputs]
    torch.cuda.synchronize()

    out = [[] for _ in inputs]
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream()  # default priority
            with torch.cuda.stream(s):
                for _ in range(10):
                    out[i].append(_linear(*inputs[i], s))
            s.synchronize()
        except Exception as exc:  # reported below, on the main thread
            errors.append(exc)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(inputs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(len(o) == 10 for o in out)
    for i in range(len(inputs)):
        for rep, res in enumerate(out[i]):
            for name, a, b in zip(("y", "dx", "dw"), res, ref[i]):
                assert torch.equal(a, b), f"shape {shapes[i]}, repetition {rep}: {name} differs"


def test_non_current_stream_owns_what_the_call_allocates():
    """A call given a stream other than the current one, with its outputs and
    workspace left for the binding to allocate: the workspace is released to
    torch's caching allocator when the wrapper returns, while the stream-K
    kernels and their fix-up still use it on that stream.  It must belong to
    that stream, so that the current stream's own allocations (made and
    written at once, below) cannot reuse it before the stream is done."""
    import torch
    M, N, K = 1024, 1536, 1024          # Wgrad and the fused backward share tiles here: a workspace is used
    assert fb.fp8_block_gemm_workspace_size(fb.FP8BLK_OP_WGRAD, M, N, K) > 0
    assert fb.fp8_block_gemm_workspace_size(fb.FP8BLK_OP_BACKWARD, M, N, K) > 0
    x = dev_bf16(synth.normal_bf16((M, K), 1.0, 82, 0))
    w = dev_bf16(synth.normal_bf16((N, K), 0.02, 82, 1))
    dy = dev_bf16(synth.normal_bf16((M, N), 1e-3, 82, 2))
    ref = _linear(x, w, dy, None)
    qx, sx, qxT, sxT = fb.fp8_quantize_dual(x)
    qdy, sdy, qdyT, sdyT = fb.fp8_quantize_dual(dy)
    ref_dw = fb.fp8_block_gemm_wgrad(qdyT, sdyT, qxT, sxT, out_dtype=torch.float32)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()              # default priority; never made current here
    nbytes = fb.fp8_block_gemm_workspace_size(fb.FP8BLK_OP_BACKWARD, M, N, K)
    for rep in range(4):
        side.wait_stream(torch.cuda.current_stream())
        y, dx, dw = _linear(x, w, dy, side)
        dw2 = fb.fp8_block_gemm_wgrad(qdyT, sdyT, qxT, sxT, out_dtype=torch.float32, stream=side)
        # the current stream allocates blocks of the workspace's size and
        # overwrites them while the side stream may still be running
        junk = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(0xFF) for _ in range(4)]
        side.synchronize()
        torch.cuda.synchronize()
        del junk
        for name, a, b in zip(("y", "dx", "dw"), (y, dx, dw), ref):
            assert torch.equal(a, b), f"repetition {rep}: {name} differs from the single-stream result"
        assert torch.equal(dw2, ref_dw), f"repetition {rep}: Wgrad differs from the single-stream result"
