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
from gpu_util import check_bf16, check_f32, dev_bf16, host, host_f32, note, require_gpu, sample_rows

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


def test_stack_call_sequence_two_layers_full_size():
    """The 28-layer stack's own call sequence at its real size, for 2 layers
    at 8192 tokens: per layer the four weights in one batched block
    quantization (no transposed copy), the forward chained through the bf16
    outputs (O input = QKV output columns 0..2047 and down input = gate/up
    output columns 0..6143, both read in place with the previous output's
    row stride, next layer input = down output), each input quantized once
    into row groups for Fprop and column groups kept for Wgrad; then the
    backward in reverse order: each dY quantized the same way, and Dgrad
    (from the weight codes as quantized) + Wgrad in one launch with the
    column-group copy retained from the forward pass.

    Every quantizer output is compared bit for bit with the oracle run on the
    GPU's own bf16 input (the retained copies after the whole backward, so
    that nothing overwrote them); every GEMM output on the edge rows and one
    random row of every 256-row band, all columns, within the GEMM tolerance
    (bf16 outputs: the rounding of the same call's fp32 result)."""
    import torch
    M = 8192
    chain = (("qkv", 4096, 2048, None), ("o", 2048, 2048, 2048), ("gate_up", 12288, 2048, None),
             ("down", 2048, 6144, 6144))
    rng = synth.rng_for(73, 99)
    f32 = torch.float32
    layers = []
    x = dev_bf16(synth.normal_bf16((M, 2048), 1.0, 73, 0))
    for layer in range(2):
        w_bits = [synth.normal_bf16((n, k), 0.02, 73, 1 + layer, li) for li, (_, n, k, _) in enumerate(chain)]
        ws = [dev_bf16(b) for b in w_bits]
        wq = fb.fp8_quantize_block_batch(ws, transpose=False)
        L = []
        for li, (name, n, k, take) in enumerate(chain):
            xin = x if take is None else x[:, :take]         # strided view of the previous output
            assert xin.shape == (M, k)
            qx, sx, qxT, sxT = fb.fp8_quantize_dual(xin)
            qw, _, sw = wq[li]
            y = fb.fp8_block_gemm_fprop(qx, sx, qw, sw)
            yf = fb.fp8_block_gemm_fprop(qx, sx, qw, sw, out_dtype=f32)      # companion: fp32 of the same call
            L.append({"name": name, "N": n, "K": k, "w_bits": w_bits[li], "x_host": host(xin.contiguous()),
                      "qx": qx, "sx": sx, "qxT": qxT, "sxT": sxT, "qw": qw, "sw": sw, "y": y, "yf": yf})
            x = y
        layers.append(L)
    torch.cuda.synchronize()
    for layer, L in reversed(list(enumerate(layers))):
        for li in reversed(range(4)):
            d = L[li]
            d["dy_bits"] = synth.normal_bf16((M, d["N"]), 1e-3, 74, layer, li)
            qdy, sdy, qdyT, sdyT = fb.fp8_quantize_dual(dev_bf16(d["dy_bits"]))
            args = (qdy, sdy, d["qw"], d["sw"], qdyT, sdyT, d["qxT"], d["sxT"])
            d["dx"], d["dw"] = fb.fp8_block_gemm_backward_w(*args)
            d["dxf"], d["dwf"] = fb.fp8_block_gemm_backward_w(*args, dx_dtype=f32, dw_dtype=f32)
            d.update(qdy=qdy, sdy=sdy, qdyT=qdyT, sdyT=sdyT)
    torch.cuda.synchronize()

    for layer, L in enumerate(layers):
        for d in L:
            tag = f"layer {layer} {d['name']}"
            ox, osx = oracle.quantize_rowgroup(d["x_host"])
            oxT, osxT = oracle.quantize_colgroup(d["x_host"])
            ow, _, osw = oracle.quantize_block(d["w_bits"], transpose=False)
            ody, osdy = oracle.quantize_rowgroup(d["dy_bits"])
            odyT, osdyT = oracle.quantize_colgroup(d["dy_bits"])
            for what, got, want in (("X row groups", (d["qx"], d["sx"]), (ox, osx)),
                                    ("X column groups kept for Wgrad", (d["qxT"], d["sxT"]), (oxT, osxT)),
                                    ("W blocks", (d["qw"], d["sw"]), (ow, osw)),
                                    ("dY row groups", (d["qdy"], d["sdy"]), (ody, osdy)),
                                    ("dY column groups", (d["qdyT"], d["sdyT"]), (odyT, osdyT))):
                assert np.array_equal(host(got[0]), want[0]), f"{tag}: {what} codes differ"
                assert np.array_equal(host(got[1]), want[1]), f"{tag}: {what} scales differ"
            n, k = d["N"], d["K"]
            for op, out, outf, nrows, ref in (
                    ("fprop", d["y"], d["yf"], M, lambda r: oracle.gemm_fprop(ox, osx, ow, osw, rows=r)),
                    ("dgrad", d["dx"], d["dxf"], M, lambda r: oracle.gemm_dgrad(ody, osdy, ow, osw, rows=r)),
                    ("wgrad", d["dw"], d["dwf"], n, lambda r: oracle.gemm_wgrad(odyT, osdyT, oxT, osxT, rows=r))):
                rows = sample_rows(nrows, rng, k=2)
                y32, _, bound = ref(rows)
                st = check_f32(host_f32(outf)[rows], y32, bound, f"{tag} {op}")
                check_bf16(host(out)[rows], host_f32(outf)[rows], y32, bound, f"{tag} {op}")
                note(f"stack {tag} {op}: {len(rows)} rows, err/bound {st['err/bound']:.2e}")
