"""Seeded synthetic inputs for the blockwise-FP8 linear layer.

This module holds input generation only -- none of the method's arithmetic --
so that the HIP path and the CPU oracle can be fed the same tensors without
sharing code.  bf16 tensors are produced as raw uint16 bit patterns.

The shapes and distributions follow the pages' workload: 8192 tokens per
micro-batch (micro-batch 2 x sequence 4096) and the Qwen3-1.7B layer layout
(hidden 2048, 16 query / 8 KV heads of 128, FFN 6144) -- "Puro-2B ... part 3/7"
section 3.1 (MBS = 2), the study notes section 2.1 (sequence 4096) and the
explainer's "Method" section (Qwen3-1.7B layout).  Activations are N(0, 1),
weights N(0, 0.02) (a usual initialisation std), output gradients N(0, 1e-3).
"""
from __future__ import annotations

import numpy as np

TOKENS = 8192

# (name, out_features N, in_features K) of one decoder layer's linears
LAYER_LINEARS = (
    ("qkv", 4096, 2048),      # 16 q heads + 2 x 8 kv heads, head_dim 128
    ("o", 2048, 2048),
    ("gate_up", 12288, 2048),  # gate and up fused, 2 x 6144
    ("down", 2048, 6144),
)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (input generation)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def rng_for(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def normal_bf16(shape, std: float, *key: int) -> np.ndarray:
    """N(0, std^2) samples drawn in fp32 with PCG64 seeded by `key`, cast to bf16."""
    x = rng_for(*key).standard_normal(shape, dtype=np.float32) * np.float32(std)
    return bf16_bits_from_f32(x)


def tiny_fprop(seed: int = 0):
    """256x256 X ~ N(0,1), 256x256 W ~ N(0,0.02)."""
    return normal_bf16((256, 256), 1.0, seed, 1, 0), normal_bf16((256, 256), 0.02, seed, 1, 1)


def single_linear(seed: int = 0, tokens: int = TOKENS):
    """X [tokens x 2048] ~ N(0,1), W (gate+up fused) [12288 x 2048] ~ N(0,0.02)."""
    return (normal_bf16((tokens, 2048), 1.0, seed, 2, 0),
            normal_bf16((12288, 2048), 0.02, seed, 2, 1))


def outlier_stress(seed: int = 0, tokens: int = TOKENS, cols: int = 2048):
    """Student-t(3) activations, 1% of channels scaled x100 (before the bf16
    cast), 0.1% of the 1x128 row groups set to +0 (after the cast).
    Returns (X bits, W bits, info dict)."""
    rng = rng_for(seed, 4, 0)
    x = rng.standard_t(3, size=(tokens, cols)).astype(np.float32)
    nch = max(1, cols // 100)
    chans = rng.choice(cols, size=nch, replace=False)
    x[:, chans] *= np.float32(100.0)
    xb = bf16_bits_from_f32(x)
    ngroups = tokens * (cols // 128)
    nz = max(1, ngroups // 1000)
    zg = rng.choice(ngroups, size=nz, replace=False)
    for g in zg:
        r, c = divmod(int(g), cols // 128)
        xb[r, c * 128:(c + 1) * 128] = 0
    w = normal_bf16((12288, cols), 0.02, seed, 4, 1)
    return xb, w, {"channels": np.sort(chans), "zero_groups": np.sort(zg)}


def decoder_layer(seed: int = 0, tokens: int = TOKENS, linears=LAYER_LINEARS):
    """Per linear: X [tokens x K] ~ N(0,1), W [N x K] ~ N(0,0.02), dY [tokens x N] ~ N(0,1e-3)."""
    out = []
    for li, (name, n, k) in enumerate(linears):
        out.append({
            "name": name, "N": n, "K": k,
            "x": normal_bf16((tokens, k), 1.0, seed, 3, 3 * li),
            "w": normal_bf16((n, k), 0.02, seed, 3, 3 * li + 1),
            "dy": normal_bf16((tokens, n), 1e-3, seed, 3, 3 * li + 2),
        })
    return out


def integer_valued_bf16(shape, lo: int, hi: int, *key: int) -> np.ndarray:
    """Uniform integers in [lo, hi] as bf16 (exact for |v| <= 256)."""
    v = rng_for(*key).integers(lo, hi + 1, size=shape).astype(np.float32)
    return bf16_bits_from_f32(v)


def device_normal_bf16(shape, std: float, seed: int, device="cuda"):
    """N(0, std^2) bf16 tensor generated on the device with torch's seeded
    Philox generator (for the large benchmark workloads)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std).to(torch.bfloat16)
