"""Pins for the oracle's scale rule and quantizers (CPU only).

The power-of-two scale follows "Puro-2B ... part 3/7" section 3.2 (third
paragraph: block scales restricted to powers of two, E8M0-like) with the
reading stated in oracle.c: the smallest 2^e with amax <= 448 * 2^e, clamped
to [-126, 127], and s = 1 for an all-zero group.  Groups are 1x128 along the
reduction dimension for activations / gradients and 128x128 for weights
(section 3.2, second paragraph).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from blockwise_fp8_linear_amd import synth


def _bits_scale_exponent(b: int) -> int:
    """Second derivation of the scale exponent, from the bf16 bit fields of
    the (non-negative) group amax: amax = (1 + m/128) * 2^E; 448 = 1.75 * 2^8,
    so e = E - 8, plus one when m/128 > 0.75 (m > 96)."""
    if b == 0:
        return 0
    field, m = b >> 7, b & 0x7F
    if field == 0:                     # subnormal amax: far below 448 * 2^-126
        return -126
    e = (field - 127) - 8 + (1 if m > 96 else 0)
    return max(-126, min(127, e))


def test_scale_rule_two_derivations_all_bf16(orc):
    for b in range(0, 0x7F80):          # all non-negative finite bf16 values
        amax = float(orc.bf16_to_f64(np.array([b], np.uint16))[0])
        assert orc.scale_exponent(amax) == _bits_scale_exponent(b), hex(b)


def test_scale_boundaries(orc):
    for e in range(-120, 121, 7):
        edge = 448.0 * 2.0 ** e
        assert orc.scale_exponent(edge) == e                       # exactly 448*2^e fits
        assert orc.scale_exponent(np.nextafter(edge, np.inf)) == e + 1
        assert orc.scale_exponent(np.nextafter(edge / 2, np.inf)) == e
    assert orc.scale_exponent(0.0) == 0
    assert orc.scale_exponent(1e-45) == -126                       # clamped


def _torch_cast(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_rowgroup_codes_against_library_cast(orc):
    """Given the scale, every code is the library's RNE cast of x / s."""
    x = synth.normal_bf16((64, 512), 1.0, 9, 9, 0)
    q, s = orc.quantize_rowgroup(x)
    xf = orc.bf16_to_f64(x)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.array_equal(q, _torch_cast(xf / srep))


def test_rowgroup_invariants(orc):
    x = synth.normal_bf16((96, 1024), 3.0, 9, 9, 1)
    x[5, 128:256] = 0                               # an all-zero group
    x[7, :128] = synth.bf16_bits_from_f32(np.full(128, -0.0, np.float32))
    q, s = orc.quantize_rowgroup(x)
    xf = orc.bf16_to_f64(x)
    dq = orc.e4m3_decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    # scales are exact powers of two
    mant, _ = np.frexp(s)
    assert np.all(mant == 0.5)
    # all-zero groups: s = 1, codes keep the sign of zero
    assert s[5, 1] == 1.0 and np.all(q[5, 128:256] == 0)
    assert s[7, 0] == 1.0 and np.all(q[7, :128] == 0x80)
    # largest decoded magnitude of a non-zero group lies in [224, 448]
    g = np.abs(orc.e4m3_decode(q)).reshape(96, 8, 128).max(axis=2)
    nz = np.abs(xf).reshape(96, 8, 128).max(axis=2) > 0
    assert np.all((g[nz] >= 224) & (g[nz] <= 448))
    # round-trip error: relative 2^-4 in the normal range, 2^-10 * s below it
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    y = np.abs(xf / srep)
    err = np.abs(dq - xf)
    normal = y >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xf[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * srep[~normal])


def _exact_group(values_bits):
    """Brute force with exact rationals: search the exponent, then the nearest
    code by exhaustive comparison, ties to even codes."""
    vals = []
    for b in values_bits:
        b = int(b)
        sign = -1 if b & 0x8000 else 1
        E, m = (b >> 7) & 0xFF, b & 0x7F
        mag = Fraction(m, 128) * Fraction(2) ** -126 if E == 0 else (1 + Fraction(m, 128)) * Fraction(2) ** (E - 127)
        vals.append((sign, mag))
    amax = max(v[1] for v in vals)
    if amax == 0:
        e = 0
    else:
        e = -200
        while amax > 448 * Fraction(2) ** e:
            e += 1
        e = max(-126, min(127, e))
    grid = []
    for c in range(0x7F):
        E, m = c >> 3, c & 7
        grid.append(Fraction(m, 512) if E == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (E - 7))
    codes = []
    for sign, mag in vals:
        y = min(mag / Fraction(2) ** e, Fraction(448))
        best = min(range(0x7F), key=lambda c: (abs(grid[c] - y), c & 1))
        codes.append(best | (0x80 if sign < 0 else 0))
    return e, codes


@pytest.mark.parametrize("case", ["random", "edges"])
def test_rowgroup_brute_force_exact(orc, case):
    rng = np.random.default_rng(11)
    if case == "random":
        x = synth.normal_bf16((3, 256), 0.7, 11, 0)
    else:
        # hand-made edges: group amax exactly 448*2^e; amax just above; values
        # that land on e4m3 subnormals and on exact ties; a bf16-subnormal group
        r0 = np.concatenate([[448.0 * 2 ** -3], rng.uniform(-50, 50, 127) * 2 ** -3])
        r1 = np.concatenate([[56.25],                    # next bf16 above 448 * 2^-3
                             (np.arange(127) - 63) * 2.0 ** -13])
        r2 = np.concatenate([[1.0], np.arange(127) * 2.0 ** -16])      # subnormal codes after /2^-8
        r3 = np.concatenate([[2.0 ** -130], -np.arange(127) * 2.0 ** -133])  # bf16 subnormals
        x = synth.bf16_bits_from_f32(np.stack([np.concatenate([r0, r1]), np.concatenate([r2, r3])]).astype(np.float32))
    q, s = orc.quantize_rowgroup(x)
    for r in range(x.shape[0]):
        for g in range(x.shape[1] // 128):
            e, codes = _exact_group(x[r, g * 128:(g + 1) * 128])
            assert s[r, g] == np.float32(2.0 ** e)
            assert list(q[r, g * 128:(g + 1) * 128]) == codes, (r, g)


def test_colgroup_is_rowgroup_of_transpose(orc):
    x = synth.normal_bf16((384, 256), 1.0, 12, 0)
    qT, sT = orc.quantize_colgroup(x)
    q2, s2 = orc.quantize_rowgroup(np.ascontiguousarray(x.T))
    assert np.array_equal(qT, q2) and np.array_equal(sT, s2)


def test_rowgroup_strided_slice(orc):
    x = synth.normal_bf16((128, 640), 1.0, 12, 1)
    q1, s1 = orc.quantize_rowgroup(x, cols=384)
    q2, s2 = orc.quantize_rowgroup(np.ascontiguousarray(x[:, :384]))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_block_transpose_identity(orc):
    w = synth.normal_bf16((256, 384), 0.02, 13, 0)
    q, qT, s = orc.quantize_block(w)
    q2, qT2, s2 = orc.quantize_block(np.ascontiguousarray(w.T))
    assert np.array_equal(qT, q2) and np.array_equal(q, qT2) and np.array_equal(s.T, s2)
    assert np.array_equal(qT, q.T)


def test_block_scale_is_max_of_rowgroup_scales(orc):
    """A block's amax is the max of its rows' 1x128 amaxes and the scale rule
    is monotone, so the block scale is the largest row-group scale inside it;
    the codes are then the library cast of w / s_block."""
    w = synth.normal_bf16((256, 256), 0.02, 13, 1)
    w[:128, 128:] = synth.bf16_bits_from_f32(np.zeros((128, 128), np.float32))
    q, _, s = orc.quantize_block(w, transpose=False)
    _, sr = orc.quantize_rowgroup(w)
    blockmax = sr.reshape(2, 128, 2).max(axis=1)
    assert np.array_equal(s, blockmax)
    assert s[0, 1] == 1.0
    srep = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    assert np.array_equal(q, _torch_cast(orc.bf16_to_f64(w) / srep))


def test_outlier_workload_paths(orc):
    """The outlier-stress inputs exercise zero groups, large scales and
    underflow to zero; the invariants must hold on them too."""
    x, _, info = synth.outlier_stress(tokens=256, cols=2048)
    q, s = orc.quantize_rowgroup(x)
    assert (s == 1.0).sum() >= 1
    assert s.max() >= 2.0 ** 0 and s.min() <= 2.0 ** -5
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    xf = orc.bf16_to_f64(x)
    assert np.array_equal(q, _torch_cast(xf / srep))
    assert np.any((q & 0x7F) == 0) and np.any((q & 0x7F) == 0x7E)
