"""Helpers shared by the GPU parity tests (host <-> device marshalling and the
GEMM tolerance gate).  No method arithmetic lives here."""
from __future__ import annotations

import sys

import numpy as np
import pytest


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import blockwise_fp8_linear_amd as fb
    fb.load_library()          # raises if the HIP library is not built: never a silent fallback


def dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def host_f32(t) -> np.ndarray:
    """A bf16 or fp32 device tensor as float32 numpy."""
    import torch
    return t.detach().float().cpu().numpy()


def sample_rows(n: int, rng, k: int = 8) -> np.ndarray:
    """Output rows for the oracle to recompute: the edges, one random row in
    every 256-row band (so every 256x256 output tile is compared, each row
    over all its columns) and k more random rows."""
    fixed = [r for r in (0, 1, 127, 128, 255, 256, n // 2 + 17, n - 129, n - 1) if 0 <= r < n]
    bands = [b + int(rng.integers(0, min(256, n - b))) for b in range(0, n, 256)]
    return np.unique(np.concatenate([fixed, bands, rng.choice(n, min(k, n), replace=False)])).astype(np.int64)


def note(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# Tolerance (the reading of "max relative error 1e-3 against the oracle's
# fp32-accumulated result"): see the module docstring of test_gpu_gemm.py.
RTOL = 1e-3


def check_f32(y: np.ndarray, y32: np.ndarray, bound: np.ndarray, what: str) -> dict:
    err = np.abs(y.astype(np.float64) - y32.astype(np.float64))
    rel_bound = float(np.max(err / np.maximum(bound, 1e-300)))
    normwise = float(err.max() / max(np.abs(y32).max(), 1e-300))
    bad = err > RTOL * bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements exceed 1e-3 * sum|terms| (worst {rel_bound:.3g})"
    assert normwise <= RTOL, f"{what}: normwise error {normwise:.3g} > 1e-3"
    return {"err/bound": rel_bound, "normwise": normwise, "exact_frac": float(np.mean(err == 0))}


def bf16_rne_np(f: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def check_bf16(ybits: np.ndarray, yf32_same_kernel: np.ndarray, y32: np.ndarray, bound: np.ndarray, what: str):
    """bf16 output: the RNE rounding of the same kernel's fp32 result, bit for
    bit, and within half a bf16 ulp (<= 2^-8 relative) plus the fp32 gate of
    the oracle's fp32 result."""
    assert np.array_equal(ybits, bf16_rne_np(yf32_same_kernel)), f"{what}: bf16 != RNE(fp32) of the same kernel"
    yb = (ybits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(yb - y32)
    lim = 2.0 ** -8 * np.abs(y32) + RTOL * bound
    assert np.all(err <= lim), f"{what}: bf16 output outside 2^-8|y| + 1e-3 sum|terms|"
