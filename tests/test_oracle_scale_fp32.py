"""Pins for the oracle's second scale rule, mode 1 (FP8BLK_SCALE_FP32; CPU only).

"Puro-2B ... part 3/7", section 3.2, third paragraph, restricts the run's
block scales to powers of two and contrasts that with the DeepSeek-V3 recipe
the grouping follows, whose scale formula the pages do not print.  The
reading implemented as a numerics variant: s = fl32(amax / 448) (1 for an
all-zero group), q = RNE-to-E4M3(fl32(x / s)) saturating at +-448.

The pins below come from outside the oracle's own arithmetic: exact rational
rounding (the correctly rounded single-precision quotient found by
bracketing), the independent nearest-code encoder, the reduction to the
power-of-two rule when amax / 448 is a power of two, the library cast, and
invariants that the rule implies.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from blockwise_fp8_linear_amd import synth

MODE = 1


def _rn32(fr: Fraction) -> np.float32:
    """The float32 nearest to the rational fr (ties to the even significand),
    by bracketing: the float32 of the nearest double is within one float32
    ulp, so the answer is it or a neighbour."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]

    def key(v):
        return (abs(Fraction(float(v)) - fr), int(np.array(v, np.float32).view(np.uint32)) & 1)

    return min(cands, key=key)


def _f64(orc, bits):
    return orc.bf16_to_f64(np.asarray(bits, np.uint16))


def test_scale_is_rounded_quotient_all_bf16(orc):
    """s = RN32(amax / 448) for every positive finite bf16 amax, subnormals
    included (the quotient then lands among the float32 subnormals)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    amax = _f64(orc, bits)
    got = np.array([orc.scale_fp32(a) for a in amax], np.float32)
    # the double quotient rounded to float32 is the correctly rounded one
    # (53 >= 2 * 24 + 2 bits), checked against exact rationals on a sample
    fast = (amax / 448.0).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), fast.view(np.uint32))
    for i in range(0, bits.size, 97):
        assert got[i] == _rn32(Fraction(float(amax[i])) / 448), hex(int(bits[i]))
    assert orc.scale_fp32(0.0) == 1.0


def _group_cases():
    """A few 1x128 groups with hand-made edges, as bf16 bits [rows, 128]."""
    rng = synth.rng_for(40, 0)
    rows = []
    rows.append(rng.standard_normal(128).astype(np.float32))                       # ordinary
    g = rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** -130)      # bf16 subnormals
    rows.append(g)
    g = rng.standard_normal(128).astype(np.float32)
    g[5] = np.float32(448.0 * 3.0)                                                  # amax 1344
    rows.append(g)
    g = np.zeros(128, np.float32)
    g[7] = -0.0
    rows.append(g)                                                                  # all zero, one -0
    g = rng.standard_normal(128).astype(np.float32) * np.float32(1e-3)
    g[0] = np.float32(-1.0)                                                         # negative amax, tiny rest
    rows.append(g)
    g = (rng.standard_normal(128) * 1e30).astype(np.float32)                        # huge values
    rows.append(g)
    return synth.bf16_bits_from_f32(np.stack(rows))


def test_codes_brute_force_exact(orc):
    """Every code equals the nearest-code encoder applied to the correctly
    rounded quotient RN32(x / s), with s = RN32(amax / 448), all by exact
    rationals."""
    x = _group_cases()
    q, s = orc.quantize_rowgroup(x, mode=MODE)
    xf = _f64(orc, x)
    for r in range(x.shape[0]):
        amax = np.max(np.abs(xf[r]))
        s_ref = np.float32(1.0) if amax == 0 else _rn32(Fraction(float(amax)) / 448)
        assert s[r, 0] == s_ref
        # s > 0, so the quotient carries x's sign (also for zeros, which the
        # rationals cannot represent signed)
        quot = np.array([np.copysign(float(_rn32(Fraction(float(v)) / Fraction(float(s_ref)))), v) for v in xf[r]])
        # the nearest-code encoder clamps at 448 itself (saturation)
        assert np.array_equal(q[r], orc.e4m3_encode_nearest(quot)), r
    assert q[3, 7] == 0x80 and np.all(np.delete(q[3], 7) == 0) and s[3, 0] == 1.0


def test_reduces_to_pow2_rule_when_amax_is_448_times_power_of_two(orc):
    """amax = 448 * 2^k: the quotient scale is exactly 2^k, which is also the
    power-of-two rule's scale, and x / 2^k is exact -- both modes must give
    the same codes and scales."""
    rng = synth.rng_for(41, 0)
    R = 96
    x = rng.uniform(-1.0, 1.0, size=(R, 256)).astype(np.float32)
    k = rng.integers(-100, 100, size=(R, 2))
    for r in range(R):
        for g in range(2):
            blk = x[r, g * 128:(g + 1) * 128]
            blk *= np.float32(2.0 ** int(k[r, g]))
            blk[rng.integers(0, 128)] = np.float32(448.0 * 2.0 ** int(k[r, g])) * rng.choice([-1, 1])
    xb = synth.bf16_bits_from_f32(x)
    q1, s1 = orc.quantize_rowgroup(xb, mode=MODE)
    q0, s0 = orc.quantize_rowgroup(xb)
    assert np.array_equal(s1, s0)
    assert np.array_equal(q1, q0)


def test_invariants(orc):
    """On the outlier workload's shape of inputs (Student-t, hot channels,
    zero groups): the two rules' scales bracket each other, every group's
    largest magnitude encodes to +-448, no code is NaN, and the round trip is
    within E4M3's half ulp plus one float32 rounding."""
    xb, w, info = synth.outlier_stress(0, tokens=256, cols=1024)
    q1, s1 = orc.quantize_rowgroup(xb, mode=MODE)
    q0, s0 = orc.quantize_rowgroup(xb)
    xf = _f64(orc, xb)
    absx = np.abs(xf).reshape(256, 8, 128)
    amax = absx.max(axis=2)
    nz = amax > 0
    # s0 / 2 < s1 <= s0 (s0 = the smallest 2^e with amax <= 448 * 2^e)
    assert np.all(s1[nz] <= s0[nz]) and np.all(s1[nz] > s0[nz] / 2)
    assert np.all(s1[~nz] == 1.0)
    codes = q1.reshape(256, 8, 128)
    is_max = (absx == amax[..., None]) & nz[..., None]
    assert np.all((codes[is_max] & 0x7F) == 0x7E)
    assert not np.any((q1 & 0x7F) == 0x7F)
    deq = orc.e4m3_decode(q1) * np.repeat(s1.astype(np.float64), 128, axis=1)
    v = xf / np.repeat(s1.astype(np.float64), 128, axis=1)
    srep = np.repeat(s1.astype(np.float64), 128, axis=1)
    err = np.abs(deq - xf)
    normal = np.abs(v) >= 2.0 ** -6
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -22) * np.abs(xf[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * srep[~normal] + 2.0 ** -22 * np.abs(xf[~normal]))


def test_codes_against_library_cast(orc):
    """Given the scale, each code is the library's RNE cast of the float32
    quotient (clamped to +-448, the saturation)."""
    x = synth.normal_bf16((64, 512), 1.0, 42, 0)
    q, s = orc.quantize_rowgroup(x, mode=MODE)
    xf = orc.bf16_to_f64(x).astype(np.float32)
    quot = xf / np.repeat(s, 128, axis=1)            # float32 division, IEEE
    quot = np.clip(quot, -448.0, 448.0).astype(np.float32)
    lib = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, lib)


def test_colgroup_and_block_identities(orc):
    x = synth.normal_bf16((256, 384), 1.0, 43, 0)
    qT, sT = orc.quantize_colgroup(x, mode=MODE)
    xt = np.ascontiguousarray(x.T)
    qr, sr = orc.quantize_rowgroup(xt, mode=MODE)
    assert np.array_equal(qT, qr) and np.array_equal(sT, sr)
    w = synth.normal_bf16((256, 384), 0.02, 43, 1)
    q, qt, s = orc.quantize_block(w, mode=MODE)
    q2, qt2, s2 = orc.quantize_block(np.ascontiguousarray(w.T), mode=MODE)
    assert np.array_equal(q, qt2) and np.array_equal(qt, q2) and np.array_equal(s, s2.T)
    # a block's scale is the quotient scale of its amax
    wf = orc.bf16_to_f64(w)
    for bi in range(2):
        for bj in range(3):
            a = np.max(np.abs(wf[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]))
            assert s[bi, bj] == _rn32(Fraction(float(a)) / 448)


def test_gemm_library_identity_with_fp32_scales(orc):
    """The contraction with non-power-of-two scales: the double result equals
    numpy's float64 product of the dequantized operands to rounding, and the
    fp32 result stays within the fp32 accumulation bound."""
    x = synth.normal_bf16((256, 512), 1.0, 44, 0)
    w = synth.normal_bf16((384, 512), 0.02, 44, 1)
    qx, sx = orc.quantize_rowgroup(x, mode=MODE)
    qw, _, sw = orc.quantize_block(w, mode=MODE)
    assert np.any(np.frexp(sx)[0] != 0.5)          # the scales really are not powers of two
    y32, y64, bnd = orc.gemm_fprop(qx, sx, qw, sw)
    dx = orc.e4m3_decode(qx) * np.repeat(sx.astype(np.float64), 128, axis=1)
    dw = orc.e4m3_decode(qw) * np.repeat(np.repeat(sw.astype(np.float64), 128, 0), 128, 1)
    ref = dx @ dw.T
    assert np.all(np.abs(y64 - ref) <= 1e-12 * bnd)
    assert np.all(np.abs(y32 - y64) <= (512 // 128 + 1) * 2.0 ** -24 * bnd + 1e-30)
