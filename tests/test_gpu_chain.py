"""The 28-layer stack's forward mechanism at reduced size: each linear's
input is (a column slice of) the previous linear's bf16 output, read in
place with its row stride, as the stack benchmark does (O input = QKV output
columns 0..2047, down input = gate/up output columns 0..6143).  Every stage
is checked against the oracle run on the same bf16 input copied to the
host: quantization bit for bit, the GEMM within the stated tolerance."""
import numpy as np
import pytest

import oracle
import blockwise_fp8_linear_amd as fb
from blockwise_fp8_linear_amd import synth
from gpu_util import check_bf16, check_f32, dev_bf16, host, host_f32, note, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_forward_chain_one_layer():
    import torch
    M = 1024
    x_bits = synth.normal_bf16((M, 2048), 1.0, 70, 0)
    chain = [("qkv", 4096, 2048, None), ("o", 2048, 2048, 2048), ("gate_up", 12288, 2048, None),
             ("down", 2048, 6144, 6144)]
    x = dev_bf16(x_bits)
    for li, (name, n, k, take) in enumerate(chain):
        xin = x if take is None else x[:, :take]           # a strided view: row stride = previous N
        assert xin.shape == (M, k)
        w_bits = synth.normal_bf16((n, k), 0.02, 70, 1 + li)
        w = dev_bf16(w_bits)
        q, s, qT, sT = fb.fp8_quantize_dual(xin)
        qw, _, sw = fb.fp8_quantize_block(w, transpose=False)
        y = fb.fp8_block_gemm_fprop(q, s, qw, sw)
        yf = fb.fp8_block_gemm_fprop(q, s, qw, sw, out_dtype=torch.float32)
        torch.cuda.synchronize()
        # the oracle on the same bf16 input (the previous stage's GPU output)
        xin_h = host(xin.contiguous()).view(np.uint16)
        q0, s0 = oracle.quantize_rowgroup(xin_h)
        qT0, sT0 = oracle.quantize_colgroup(xin_h)
        assert np.array_equal(host(q), q0) and np.array_equal(host(s), s0), f"{name}: row groups differ"
        assert np.array_equal(host(qT), qT0) and np.array_equal(host(sT), sT0), f"{name}: column groups differ"
        ow, _, osw = oracle.quantize_block(w_bits, transpose=False)
        rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], synth.rng_for(70, li).choice(M, 12, replace=False)]))
        y32, _, bound = oracle.gemm_fprop(q0, s0, ow, osw, rows=rows)
        st = check_f32(host_f32(yf)[rows], y32, bound, f"chain {name}")
        check_bf16(host(y)[rows], host_f32(yf)[rows], y32, bound, f"chain {name}")
        note(f"chain {name}: {st}")
        x = y
