#!/usr/bin/env python3
"""Benchmark of the blockwise-FP8 linear layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input.
Default workload ("layer"): one decoder layer's four linears (QKV 2048->4096,
O 2048->2048, gate/up 2048->12288, down 6144->2048) at 8192 tokens: the four
weights block-quantized in one launch (no transposed copy: Dgrad reads the
codes as quantized), then per linear one-pass row-group + column-group
quantization of X, Fprop, one-pass quantization of dY, and Dgrad + Wgrad in
one fused launch -- 2.474 TFLOP of FP8 GEMM per step.  --separate-quant,
--separate-wquant, --transposed-weights and --separate-bwd switch each of
these back to its plain form.

Other workloads: "linear" (the 8192 x 2048 -> 12288 gate/up linear, quantize
+ Fprop only) and "stack28" (28 decoder layers, forward chained through the
layer outputs, then backward, timed against the same GEMMs in bf16).

Prints ONE JSON line.  Inputs are seeded synthetic tensors generated on the
device before timing.  Durations come from HIP events recorded on the launch
stream: around every launch in an untimed breakdown pass; in every 4th
timed step, around the dominant kernel's launches and at the step's start
and end.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "blockwise-FP8 linear TFLOP/s (fprop+dgrad+wgrad, 8192 tok) + % FP8 peak"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
TOKENS = 8192
LINEARS = (("qkv", 4096, 2048), ("o", 2048, 2048), ("gate_up", 12288, 2048), ("down", 2048, 6144))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
KERNEL_SOURCES = ("blockwise_fp8_linear_amd/csrc/gemm_mx.hip", "blockwise_fp8_linear_amd/csrc/gemm.hip",
                  "blockwise_fp8_linear_amd/csrc/quant.hip", "blockwise_fp8_linear_amd/csrc/fp8blk_device.h")


def kernel_of(kind, algo):
    """The kernel function a timed launch runs (Fprop and Dgrad from the
    transposed weight copy share one)."""
    fast = algo in ("default", "scaled")
    bt = "true" if DGRAD_W else "false"
    if kind == "gemm_fprop" or (kind == "gemm_dgrad" and not DGRAD_W):
        return "gemm_mx_kernel<false, false>" if fast else "gemm_kernel<promote, weight-block scales>"
    if kind == "gemm_dgrad":
        return "gemm_mx_kernel<false, true>" if fast else "gemm_kernel<promote, weight-block scales, W as quantized>"
    if kind == "gemm_bwd":
        return f"gemm_mx_bwd_kernel<{bt}> (+ bwd_fixup_kernel)"
    if kind == "gemm_wgrad":
        return ("gemm_mx_streamk_kernel<true> (+ sk_fixup_kernel)" if fast
                else "gemm_sk_kernel<promote, row scales> (+ gk_fixup_kernel)")
    return kind + "_kernel"


def sources_digest():
    """Digest of the kernel sources' code: comments and whitespace are
    dropped, so that a comment-only edit keeps the measured traffic valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, algo):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when there is none or the kernels changed since.  A
    label "a (+ b)" is a call that launches a and sometimes b: b's bytes are
    counted in the proportion of its dispatches to a's."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.loads(f.read().split("BEGIN-JSON", 1)[1].split("END-JSON", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("sources_digest") != sources_digest() or rec.get("workload") != workload or rec.get("algo") != algo:
        return None
    names = [n.strip() for n in kernel.replace("(+", "+").replace(")", "").split("+")]
    ks = rec.get("kernels", {})
    if any(n not in ks for n in names):
        return None
    main = ks[names[0]]
    return round(sum(ks[n]["hbm_bytes_per_launch"] * ks[n]["dispatches"] / main["dispatches"] for n in names))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed steps run right before the timed ones (at least 1), after one step that counts "
                         "the launches and the three-step breakdown pass")
    ap.add_argument("--workload", choices=("layer", "linear", "stack28"), default="layer")
    ap.add_argument("--algo", choices=("default", "promote", "scaled"), default="default")
    ap.add_argument("--scale", choices=("pow2", "fp32"), default="pow2",
                    help="scale rule of every quantizer: power of two (the pages' run) or amax / 448 "
                         "(FP8BLK_SCALE_FP32, which the GEMMs take only through the promote algorithm)")
    ap.add_argument("--separate-quant", action="store_true",
                    help="quantize X and dY with the separate row-group and column-group kernels "
                         "instead of the one-pass kernel")
    ap.add_argument("--separate-bwd", action="store_true",
                    help="run Dgrad and Wgrad as two calls instead of fp8_block_gemm_backward")
    ap.add_argument("--transposed-weights", action="store_true",
                    help="Dgrad reads a transposed weight copy written by the block quantizer (default: Dgrad "
                         "reads the weight codes as quantized, and no copy is written)")
    ap.add_argument("--separate-wquant", action="store_true",
                    help="quantize each weight in its own launch instead of one batched launch per layer")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip measuring the on-box MFMA and copy ceilings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--graph", action="store_true",
                    help="replay every timed step from one HIP graph captured after the warm-up (the host then "
                         "enqueues one graph per step); the roofline's kernel durations then come from eager "
                         "steps run right after the timed ones")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (a known-size reference for HBM byte counters)")
    args = ap.parse_args()
    args.warmup = max(1, args.warmup)
    return args


class Timer:
    """Events around launches, on the stream the library launches on.  The
    events are created up front (creating one costs far more host time than
    recording it).  Recording one costs GPU time too, so a Timer can be
    limited to some kinds of launch (`only`); a disabled Timer only counts
    launches."""

    def __init__(self, torch, enabled, n_launches=0, only=None):
        self.torch = torch
        self.enabled = enabled
        self.only = only
        self.count = 0
        self.recs = []
        self.pool = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(n_launches)] if enabled else []

    def run(self, kind, flops, nbytes, fn):
        self.count += 1
        if not self.enabled or (self.only is not None and kind not in self.only):
            return fn()
        s, e = self.pool[len(self.recs)]
        s.record()
        out = fn()
        e.record()
        self.recs.append((kind, flops, nbytes, s, e))
        return out

    def summary(self):
        agg = {}
        for kind, flops, nbytes, s, e in self.recs:
            ms = s.elapsed_time(e)
            a = agg.setdefault(kind, {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
            a["launches"] += 1
            a["ms"] += ms
            a["flops"] += flops
            a["bytes"] += nbytes
        return agg


def build_layer(torch, fb, synth, seed, linears=LINEARS, x_in=None):
    """Allocate inputs and every output / scratch buffer for one layer."""
    L = []
    for li, (name, n, k) in enumerate(linears):
        d = {"name": name, "N": n, "K": k}
        d["x"] = synth.device_normal_bf16((TOKENS, k), 1.0, seed * 1000 + 3 * li)
        d["w"] = synth.device_normal_bf16((n, k), 0.02, seed * 1000 + 3 * li + 1)
        d["dy"] = synth.device_normal_bf16((TOKENS, n), 1e-3, seed * 1000 + 3 * li + 2)
        u8, f32 = torch.uint8, torch.float32
        d["qx"] = torch.empty((TOKENS, k), dtype=u8, device="cuda")
        d["sx"] = torch.empty((TOKENS, k // 128), dtype=f32, device="cuda")
        d["qxT"] = torch.empty((k, TOKENS), dtype=u8, device="cuda")
        d["sxT"] = torch.empty((k, TOKENS // 128), dtype=f32, device="cuda")
        d["qw"] = torch.empty((n, k), dtype=u8, device="cuda")
        d["qwT"] = None if DGRAD_W else torch.empty((k, n), dtype=u8, device="cuda")
        d["sw"] = torch.empty((n // 128, k // 128), dtype=f32, device="cuda")
        d["qdy"] = torch.empty((TOKENS, n), dtype=u8, device="cuda")
        d["sdy"] = torch.empty((TOKENS, n // 128), dtype=f32, device="cuda")
        d["qdyT"] = torch.empty((n, TOKENS), dtype=u8, device="cuda")
        d["sdyT"] = torch.empty((n, TOKENS // 128), dtype=f32, device="cuda")
        d["y"] = torch.empty((TOKENS, n), dtype=torch.bfloat16, device="cuda")
        d["dx"] = torch.empty((TOKENS, k), dtype=torch.bfloat16, device="cuda")
        d["dw"] = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
        ws = max(fb.fp8_block_gemm_workspace_size(fb.FP8BLK_OP_WGRAD, TOKENS, n, k),
                 fb.fp8_block_gemm_workspace_size(fb.FP8BLK_OP_BACKWARD, TOKENS, n, k))
        d["ws"] = torch.empty(max(ws, 16), dtype=u8, device="cuda")
        L.append(d)
    return L


def qbytes(rows, cols):
    return rows * cols * 3 + rows * (cols // 128) * 4


def dual_bytes(rows, cols):
    return rows * cols * 4 + 2 * rows * (cols // 128) * 4


# True: one pass writes both the row-group and the column-group copy of X and
# of dY; False: two passes (the separate row-group and column-group kernels).
DUAL = True
# True: Dgrad and Wgrad of a linear in one call (fp8_block_gemm_backward);
# False: the two separate calls.
FUSED_BWD = True
# True: a layer's four weights quantized in one launch; False: one launch each.
BATCH_W = True
# Scale rule of every quantizer call (FP8BLK_SCALE_POW2 or FP8BLK_SCALE_FP32).
SCALE_MODE = 0
# True: Dgrad reads the weight codes W[n][k] as quantized (no transposed copy
# written); False: the block quantizer also writes W^T's codes for Dgrad.
DGRAD_W = True


def quantize_both(fb, T, x, q, s, qT, sT):
    rows, cols = x.shape
    if DUAL:
        T.run("quant_dual", 0, dual_bytes(rows, cols),
              lambda: fb.fp8_quantize_dual(x, q=q, s=s, qT=qT, sT=sT, scale_mode=SCALE_MODE))
    else:
        T.run("quant_rowgroup", 0, qbytes(rows, cols),
              lambda: fb.fp8_quantize_rowgroup(x, q=q, s=s, scale_mode=SCALE_MODE))
        T.run("quant_colgroup", 0, qbytes(rows, cols),
              lambda: fb.fp8_quantize_colgroup(x, qT=qT, sT=sT, scale_mode=SCALE_MODE))


def quantize_weights(fb, T, L):
    """All the weights of a layer (with their transposed copies), known when
    the step starts: one batched launch, or one launch per weight."""
    per = 3 if DGRAD_W else 4     # bytes per weight: bf16 read, codes (and the transposed codes) written
    if BATCH_W:
        nbytes = sum(d["N"] * d["K"] * per + (d["N"] // 128) * (d["K"] // 128) * 4 for d in L)
        T.run("quant_block_batch", 0, nbytes,
              lambda: fb.fp8_quantize_block_batch([d["w"] for d in L],
                                                  outs=[(d["qw"], None if DGRAD_W else d["qwT"], d["sw"]) for d in L],
                                                  scale_mode=SCALE_MODE))
    else:
        for d in L:
            n, k = d["N"], d["K"]
            T.run("quant_block", 0, n * k * per + (n // 128) * (k // 128) * 4,
                  lambda d=d: fb.fp8_quantize_block(d["w"], transpose=not DGRAD_W, q=d["qw"],
                                                    qT=None if DGRAD_W else d["qwT"], s=d["sw"],
                                                    scale_mode=SCALE_MODE))


def fwd_linear(fb, T, d, algo, x=None):
    n, k = d["N"], d["K"]
    x = d["x"] if x is None else x
    quantize_both(fb, T, x, d["qx"], d["sx"], d["qxT"], d["sxT"])
    T.run("gemm_fprop", 2.0 * TOKENS * n * k, 0,
          lambda: fb.fp8_block_gemm(fb.FP8BLK_OP_FPROP, d["qx"], d["sx"], d["qw"], d["sw"], TOKENS, n, k,
                                    algo=algo, out=d["y"], scale_mode=SCALE_MODE))
    return d["y"]


def bwd_linear(fb, T, d, algo):
    n, k = d["N"], d["K"]
    quantize_both(fb, T, d["dy"], d["qdy"], d["sdy"], d["qdyT"], d["sdyT"])
    if FUSED_BWD and algo == fb.FP8BLK_ALGO_DEFAULT:
        bwd = fb.fp8_block_gemm_backward_w if DGRAD_W else fb.fp8_block_gemm_backward
        T.run("gemm_bwd", 2 * 2.0 * TOKENS * n * k, 0,
              lambda: bwd(d["qdy"], d["sdy"], d["qw"] if DGRAD_W else d["qwT"], d["sw"], d["qdyT"], d["sdyT"],
                          d["qxT"], d["sxT"], dx=d["dx"], dw=d["dw"], workspace=d["ws"]))
        return
    T.run("gemm_dgrad", 2.0 * TOKENS * n * k, 0,
          lambda: fb.fp8_block_gemm(fb.FP8BLK_OP_DGRAD_W if DGRAD_W else fb.FP8BLK_OP_DGRAD, d["qdy"], d["sdy"],
                                    d["qw"] if DGRAD_W else d["qwT"], d["sw"], TOKENS, n, k, algo=algo, out=d["dx"],
                                    scale_mode=SCALE_MODE))
    T.run("gemm_wgrad", 2.0 * TOKENS * n * k, 0,
          lambda: fb.fp8_block_gemm(fb.FP8BLK_OP_WGRAD, d["qdyT"], d["sdyT"], d["qxT"], d["sxT"], TOKENS, n, k,
                                    algo=algo, out=d["dw"], workspace=d["ws"], scale_mode=SCALE_MODE))


def layer_step(fb, T, L, algo):
    quantize_weights(fb, T, L)
    for d in L:
        fwd_linear(fb, T, d, algo)
    for d in reversed(L):
        bwd_linear(fb, T, d, algo)


def linear_step(fb, T, d, algo):
    n, k = d["N"], d["K"]
    T.run("quant_rowgroup", 0, qbytes(TOKENS, k),
          lambda: fb.fp8_quantize_rowgroup(d["x"], q=d["qx"], s=d["sx"], scale_mode=SCALE_MODE))
    T.run("quant_block", 0, n * k * 3 + (n // 128) * (k // 128) * 4,
          lambda: fb.fp8_quantize_block(d["w"], transpose=False, q=d["qw"], s=d["sw"], scale_mode=SCALE_MODE))
    T.run("gemm_fprop", 2.0 * TOKENS * n * k, 0,
          lambda: fb.fp8_block_gemm(fb.FP8BLK_OP_FPROP, d["qx"], d["sx"], d["qw"], d["sw"], TOKENS, n, k,
                                    algo=algo, out=d["y"], scale_mode=SCALE_MODE))


def stack_step(fb, T, layers, algo):
    """28 layers: forward chained (O input = QKV output columns 0..2047, gate/up
    input = O output, down input = gate/up output columns 0..6143, next layer
    input = down output), then backward with each linear's own dY and the
    column-group copy of its input kept from the forward pass."""
    x = layers[0][0]["x"]
    for L in layers:
        quantize_weights(fb, T, L)
        qkv, o, gu, dn = L
        y = fwd_linear(fb, T, qkv, algo, x)
        y = fwd_linear(fb, T, o, algo, y[:, :2048])
        y = fwd_linear(fb, T, gu, algo, y)
        x = fwd_linear(fb, T, dn, algo, y[:, :6144])
    for L in reversed(layers):
        for d in reversed(L):
            bwd_linear(fb, T, d, algo)


def gemm_flops(linears):
    return sum(3 * 2.0 * TOKENS * n * k for _, n, k in linears)


def bf16_baseline(torch, linears, reps, steps=5):
    """The same GEMM shapes as the FP8 step, in bf16 via torch.matmul."""
    mats = []
    for _, n, k in linears:
        x = torch.randn(TOKENS, k, device="cuda", dtype=torch.bfloat16)
        w = torch.randn(n, k, device="cuda", dtype=torch.bfloat16)
        dy = torch.randn(TOKENS, n, device="cuda", dtype=torch.bfloat16)
        mats.append((x, w.t().contiguous(), dy, w, dy.t().contiguous()))

    def one():
        for _ in range(reps):
            for x, wt, dy, w, dyt in mats:
                torch.matmul(x, wt)
                torch.matmul(dy, w)
                torch.matmul(dyt, x)

    one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    return dt, gemm_flops(linears) * reps / dt / 1e12


def onbox_ceilings(torch):
    """What this machine sustains, measured here: the GEMM kernels' MFMA work
    alone (libfp8probe: the same block-scaled 32x32x64 FP8 instruction, one
    wave per SIMD, 16 accumulators, random codes, no memory traffic) and HBM
    streaming (libfp8probe's copy and read kernels over 1 GiB: 16-byte
    non-temporal accesses, eight in flight per lane; the copy counts read +
    write bytes, the quantizers' 1:1 mix), besides torch's own copy."""
    import ctypes
    from blockwise_fp8_linear_amd.build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    lib.fp8probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.fp8probe_mfma.restype = ctypes.c_int
    lib.fp8probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.fp8probe_mfma_flops.restype = ctypes.c_double
    wgs, iters = 256, 20000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn, reps=5):
        fn()
        best = None
        for _ in range(reps):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            e.synchronize()
            ms = s.elapsed_time(e)
            best = ms if best is None else min(best, ms)
        return best * 1e-3

    def mfma():
        if lib.fp8probe_mfma(wgs, iters, 12345, out.data_ptr(), stream) != 0:
            raise RuntimeError("fp8probe_mfma failed")
    t = timed(mfma)
    mfma_tf = lib.fp8probe_mfma_flops(wgs, iters) / t / 1e12
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 256)
    dst = torch.empty_like(src)
    lib.fp8probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.fp8probe_stream.restype = ctypes.c_int

    def stream_probe(mode):
        if lib.fp8probe_stream(mode, src.data_ptr(), dst.data_ptr(), n, 4096, stream) != 0:
            raise RuntimeError("fp8probe_stream failed")
    copy_gbs = 2 * n / timed(lambda: stream_probe(0)) / 1e9
    read_gbs = n / timed(lambda: stream_probe(1)) / 1e9
    torch_copy_gbs = 2 * n / timed(lambda: dst.copy_(src)) / 1e9
    return {"mfma_fp8_TFLOP/s": round(mfma_tf, 1), "copy_GB/s": round(copy_gbs, 1), "read_GB/s": round(read_gbs, 1),
            "torch_copy_GB/s": round(torch_copy_gbs, 1),
            "what": "best of 5: block-scaled FP8 MFMA loop (GEMM layout, random codes, no memory); a streaming "
                    "copy (read + write bytes) and a streaming read over 1 GiB (16-byte non-temporal accesses, "
                    "8 in flight per lane, 4096 workgroups); torch's device copy of the same buffer"}


def cpu_baseline(budget_s, mode=0):
    """The CPU oracle, as it stands, on a bounded sample of the layer
    workload, scaled to a whole-step rate: the oracle quantizes every
    operand of the four linears at full size (timed), then computes sampled
    output rows of each linear's fprop, dgrad and wgrad (timed) in rounds
    until the time budget is spent; GEMM time is scaled by total rows /
    sampled rows."""
    import numpy as np
    import oracle
    from blockwise_fp8_linear_amd import synth

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rows_per = max(8, threads)
    rng = np.random.default_rng(7)
    t_q = 0.0
    ops = []
    for li, (name, n, k) in enumerate(LINEARS):
        x = synth.normal_bf16((TOKENS, k), 1.0, 0, 3, 3 * li)
        w = synth.normal_bf16((n, k), 0.02, 0, 3, 3 * li + 1)
        dy = synth.normal_bf16((TOKENS, n), 1e-3, 0, 3, 3 * li + 2)
        t0 = time.perf_counter()
        qx, sx = oracle.quantize_rowgroup(x, mode=mode)
        qxT, sxT = oracle.quantize_colgroup(x, mode=mode)
        qw, _, sw = oracle.quantize_block(w, transpose=False, mode=mode)
        qdy, sdy = oracle.quantize_rowgroup(dy, mode=mode)
        qdyT, sdyT = oracle.quantize_colgroup(dy, mode=mode)
        t_q += time.perf_counter() - t0
        ops.append({"rows": TOKENS, "t": 0.0, "done": 0, "flops": 2.0 * TOKENS * n * k,
                    "fn": lambda r, a=(qx, sx, qw, sw): oracle.gemm_fprop(*a, rows=r)})
        ops.append({"rows": TOKENS, "t": 0.0, "done": 0, "flops": 2.0 * TOKENS * n * k,
                    "fn": lambda r, a=(qdy, sdy, qw, sw): oracle.gemm_dgrad(*a, rows=r)})
        ops.append({"rows": n, "t": 0.0, "done": 0, "flops": 2.0 * TOKENS * n * k,
                    "fn": lambda r, a=(qdyT, sdyT, qxT, sxT): oracle.gemm_wgrad(*a, rows=r)})
    t_spent = t_q
    rounds = 0
    while True:
        for op in ops:
            r = rng.choice(op["rows"], rows_per, replace=False)
            t0 = time.perf_counter()
            op["fn"](r)
            op["t"] += time.perf_counter() - t0
            op["done"] += rows_per
        rounds += 1
        t_spent = t_q + sum(op["t"] for op in ops)
        if t_spent > budget_s:
            break
    t_est = t_q + sum(op["t"] * op["rows"] / op["done"] for op in ops)
    flops = sum(op["flops"] for op in ops)
    return {
        "value": round(flops / t_est / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"one decoder layer's four linears at 8192 tokens: full-size oracle quantization of X, W and "
                   f"dY (row, column and block groups), plus {rounds} x {rows_per} sampled output rows of each "
                   f"fprop/dgrad/wgrad, GEMM time scaled to all rows; {t_spent:.1f} s of CPU work, est. "
                   f"{t_est:.0f} s per full step, {platform.processor() or platform.machine()}, "
                   f"{os.cpu_count()} logical CPUs"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (--gpus {args.gpus} requested); "
              "across GPUs only the Wgrad gradients would need an all-reduce; it is not implemented", file=sys.stderr)
        sys.exit(2)
    import torch
    import blockwise_fp8_linear_amd as fb
    from blockwise_fp8_linear_amd import synth

    fb.load_library()
    torch.cuda.set_device(0)
    global DUAL, FUSED_BWD, BATCH_W, SCALE_MODE, DGRAD_W
    DGRAD_W = not args.transposed_weights
    DUAL = not args.separate_quant
    FUSED_BWD = not args.separate_bwd
    BATCH_W = not args.separate_wquant
    if args.scale == "fp32":
        # amax / 448 scales are not powers of two: only the promote GEMM takes them
        if args.algo == "scaled":
            print("bench.py: --scale fp32 needs the promote algorithm (the block-scaled MFMA applies "
                  "power-of-two scales only)", file=sys.stderr)
            sys.exit(2)
        args.algo = "promote"
        SCALE_MODE = fb.FP8BLK_SCALE_FP32
    algo = {"default": fb.FP8BLK_ALGO_DEFAULT, "promote": fb.FP8BLK_ALGO_PROMOTE,
            "scaled": fb.FP8BLK_ALGO_SCALED_MFMA}[args.algo]

    if args.workload == "layer":
        L = build_layer(torch, fb, synth, 0)
        step = lambda T: layer_step(fb, T, L, algo)
        step_flops = gemm_flops(LINEARS)
        reps, linears = 1, LINEARS
        desc = "one decoder layer's linears (QKV, O, gate/up, down), fprop+dgrad+wgrad, 8192 tokens"
    elif args.workload == "linear":
        L = build_layer(torch, fb, synth, 0, linears=(("gate_up", 12288, 2048),))
        step = lambda T: linear_step(fb, T, L[0], algo)
        step_flops = 2.0 * TOKENS * 12288 * 2048
        reps, linears = None, None
        desc = "gate/up linear 8192x2048 -> 12288: quantize + fprop"
    else:
        layers = [build_layer(torch, fb, synth, s) for s in range(28)]
        step = lambda T: stack_step(fb, T, layers, algo)
        step_flops = 28 * gemm_flops(LINEARS)
        reps, linears = 28, LINEARS
        desc = "28 decoder layers' linears, forward chained then backward, 8192 tokens"

    null = Timer(torch, False)
    step(null)  # counts the launches of one step
    per_step = null.count
    torch.cuda.synchronize()

    # Breakdown pass (untimed): events around every launch, for the per-kind
    # figures and to find the dominant kernel.
    nb = 3
    B = Timer(torch, True, per_step * nb)
    for _ in range(nb):
        step(B)
    torch.cuda.synchronize()
    agg = B.summary()
    breakdown = {}
    for kind, a in agg.items():
        avg_ms = a["ms"] / a["launches"]
        e = {"launches_per_step": a["launches"] // nb, "avg_ms": round(avg_ms, 5),
             "ms_per_step": round(a["ms"] / nb, 4)}
        if a["flops"]:
            e["TFLOP/s_incl_event_overhead"] = round(a["flops"] / (a["ms"] * 1e-3) / 1e12, 1)
        if a["bytes"]:
            e["GB/s_incl_event_overhead"] = round(a["bytes"] / (a["ms"] * 1e-3) / 1e9, 1)
        breakdown[kind] = e
    gemm_kinds = [k for k in agg if k.startswith("gemm")]
    gemm_ms = sum(agg[k]["ms"] for k in gemm_kinds)
    gemm_flops_t = sum(agg[k]["flops"] for k in gemm_kinds)
    by_kernel = {}
    for kind, a in agg.items():
        b = by_kernel.setdefault(kernel_of(kind, args.algo), {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
        for f in b:
            b[f] += a[f]
    dom = max(by_kernel, key=lambda k: by_kernel[k]["ms"])
    dom_kinds = {k for k in agg if kernel_of(k, args.algo) == dom}

    # Timed steps: events only around the dominant kernel's launches (the
    # roofline's durations are measured here, live).
    # An event at every step boundary on the stream the steps run on gives the
    # spread of single-step times (recording an event does not synchronise).
    # The host enqueues a step in roughly 0.3-1.2 ms against about 1.35 ms of
    # GPU time, so a pause of the Python garbage collector could starve the
    # GPU: collect now and keep it off while the timed steps are enqueued.
    # Events cost GPU time (about 2.6 us each), so only every SAMPLE-th timed
    # step carries them: one at its start and end (the single-step spread)
    # and a pair around each of the dominant kernel's launches (the
    # roofline's durations).  The other steps run bare.
    SAMPLE = 4
    n_sampled = (args.steps + SAMPLE - 1) // SAMPLE
    T = Timer(torch, True, per_step * n_sampled, only=dom_kinds)
    bare = Timer(torch, False)
    bounds = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_sampled)]
    graph = None
    if args.graph:
        # capture one whole step (every call only enqueues on the current
        # stream, which is the capture stream here); replays run all of it
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(Timer(torch, False))
        graph.replay()
        torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    # The warm-up steps run last, right before the timed ones: the chip's
    # clock falls while it idles (the host work above takes milliseconds) and
    # takes several steps to come back, so warm-up steps run earlier left the
    # first timed steps 10-25% slow (measured: 1.355-1.361 ms per step over
    # 50 steps against 1.328-1.330 with the warm-up here).
    for _ in range(args.warmup):
        if graph is not None:
            graph.replay()
        else:
            step(bare)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % SAMPLE == 0:
            b0, b1 = bounds[i // SAMPLE]
            b0.record()
            if graph is not None:
                graph.replay()
            else:
                step(T)
            b1.record()
        elif graph is not None:
            graph.replay()
        else:
            step(bare)
    enqueued = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    if graph is not None:
        # events cannot surround single kernels inside a replay: the dominant
        # kernel's durations come from as many eager steps, right after
        for i in range(n_sampled):
            step(T)
        torch.cuda.synchronize()
    per_step_ms = sorted(b0.elapsed_time(b1) for b0, b1 in bounds)

    def pct(p):
        return round(per_step_ms[min(len(per_step_ms) - 1, int(p * len(per_step_ms)))], 4)
    ms = wall / args.steps * 1e3
    value = step_flops / (ms * 1e-3) / 1e12

    a = {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0}
    for kind, x in T.summary().items():
        for f in a:
            a[f] += x[f]
    avg_s = a["ms"] / a["launches"] * 1e-3
    traffic = measured_traffic(dom, args.workload, args.algo)
    if a["flops"]:
        ach = a["flops"] / a["launches"] / avg_s / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                "avg_launch_ms": round(avg_s * 1e3, 5), "launches": a["launches"]}
    else:
        ach = a["bytes"] / a["launches"] / avg_s / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                "avg_launch_ms": round(avg_s * 1e3, 5), "launches": a["launches"]}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms_spread": {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9),
                           "mean": round(sum(per_step_ms) / len(per_step_ms), 4),
                           "host_enqueue_ms": round(enqueued / args.steps * 1e3, 4),
                           "what": "single-step times of every 4th timed step (events at its start and end" +
                                   ("" if args.graph else
                                    "; those steps also carry the events around the dominant kernel's launches") +
                                   "); host_enqueue_ms: host time per timed step to enqueue the steps"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": desc, "name": args.workload, "tokens": TOKENS, "algo": args.algo,
                   "scale": "power of two" if args.scale == "pow2" else "fp32 amax/448",
                   "quantizer": "separate" if args.separate_quant else "one-pass",
                   "backward": "separate" if args.separate_bwd else "fused",
                   "weight_quant": "per weight" if args.separate_wquant else "batched per layer",
                   "dgrad_weights": "transposed copy" if args.transposed_weights else "codes as quantized",
                   "launch": "one HIP graph per step" if args.graph else "eager",
                   "gemm_tflop_per_step": round(step_flops / 1e12, 4)},
        "pct_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "gemm_only_TFLOP/s": round(gemm_flops_t / (gemm_ms * 1e-3) / 1e12, 1) if gemm_ms else None,
        "roofline": roof,
        "breakdown": breakdown,
        "breakdown_note": "per-kind event times from 3 untimed steps with events around every launch; a "
                          "pair of events adds a few microseconds to each launch (the first launch of a step "
                          "can also include host enqueue time), so these per-kind rates understate the "
                          "kernels, short ones most: the kernel traces in profiles/ give their durations. The "
                          "roofline comes from the dominant kernel's own events in the timed steps" +
                          (" (with --graph: in as many eager steps right after them)" if args.graph else ""),
        "sources_digest": sources_digest(),
    }
    if not args.no_ceilings:
        ceil = onbox_ceilings(torch)
        out["onbox_ceilings"] = ceil
        key = "mfma_fp8_TFLOP/s" if roof["unit"] == "TFLOP/s" else "copy_GB/s"
        roof["onbox_ceiling"] = ceil[key]
        roof["frac_of_onbox"] = round(roof["achieved"] / ceil[key], 4)
    if linears is not None and not args.no_bf16_baseline:
        dt, tf = bf16_baseline(torch, linears, reps if args.workload != "stack28" else 28)
        out["bf16_baseline"] = {"ms_per_step": round(dt * 1e3, 3), "TFLOP/s": round(tf, 1),
                                "fp8_over_bf16": round(dt * 1e3 / ms, 3),
                                "what": "the same GEMMs in bf16 via torch.matmul (hipBLASLt), no quantization"}
    if args.copy_calibration:
        src = torch.empty(256 * 1024 * 1024, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration"] = {"bytes_read": src.numel() * 2, "bytes_written": dst.numel() * 2, "launches": 3}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget_s, mode=SCALE_MODE)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
