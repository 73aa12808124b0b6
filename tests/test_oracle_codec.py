"""Pins for the oracle's E4M3 codec (CPU only).

Each check ties the oracle to something other than itself: the printed E4M3
table that the pages' FP8 section cites, an independent library decoder and
encoder (torch.float8_e4m3fn), a second encoder written as a search, and
exhaustive enumeration.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_table1.txt")


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_encode(v: np.ndarray) -> np.ndarray:
    # torch casts RNE; values beyond 448 become NaN there, so clamp first
    t = torch.from_numpy(np.clip(v, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_golden_table_values(orc):
    n = 0
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code_s, val_s = line.split()
        code = int(code_s, 16)
        got = float(orc.e4m3_decode(np.array([code], np.uint8))[0])
        if val_s == "nan":
            assert math.isnan(got), hex(code)
        else:
            want = float(val_s)
            assert got == want, (hex(code), got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, want), hex(code)
            if not math.isnan(want):
                assert orc.e4m3_encode(np.array([want]))[0] == code
        n += 1
    assert n >= 10


def test_decode_all_codes_against_library(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    lib = _torch_decode(codes)
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(lib))
    assert nan_ours.sum() == 2 and nan_ours[0x7F] and nan_ours[0xFF]
    assert np.array_equal(ours[~nan_ours], lib[~nan_ours])
    # sign bit of zero
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_finite_codes_count_and_monotone(orc):
    pos = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)           # strictly increasing over 0x00..0x7E
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9


def test_round_trip_all_finite_codes(orc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = orc.e4m3_decode(codes)
    assert np.array_equal(orc.e4m3_encode(vals), codes)
    assert np.array_equal(orc.e4m3_encode_nearest(vals), codes)


def test_midpoints_round_to_even(orc):
    pos = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2          # exact in double
    lo = np.arange(0x7E)
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(orc.e4m3_encode(mids), even)
    assert np.array_equal(orc.e4m3_encode(-mids), even | 0x80)
    below = np.nextafter(mids, -np.inf)
    above = np.nextafter(mids, np.inf)
    assert np.array_equal(orc.e4m3_encode(below), lo.astype(np.uint8))
    assert np.array_equal(orc.e4m3_encode(above), (lo + 1).astype(np.uint8))


def test_saturation_and_signs(orc):
    v = np.array([448.0, 449.0, 464.0, 480.0, 1e30, np.inf, -448.5, -np.inf, -0.0, -1e-30, 2.0 ** -10, 3 * 2.0 ** -10])
    want = np.array([0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x80, 0x00, 0x02], np.uint8)
    assert np.array_equal(orc.e4m3_encode(v), want)
    assert np.array_equal(orc.e4m3_encode_nearest(v), want)


def test_exhaustive_bf16_times_powers_of_two(orc):
    """Every finite bf16 value times 2^j, j in [-30, 30]: the two oracle
    encoders agree bit for bit, and agree with the library cast (on values
    clamped to +-448, which the library does not saturate)."""
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32).astype(np.float64)
    x = x[np.isfinite(x)]
    vals = np.concatenate([x * 2.0 ** j for j in range(-30, 31)])
    a = orc.e4m3_encode(vals)
    b = orc.e4m3_encode_nearest(vals)
    assert np.array_equal(a, b)
    c = _torch_encode(vals)
    # torch keeps -0 for negative values that round to zero, as we do
    assert np.array_equal(a, c)


def test_rounding_mode(orc):
    assert orc.rounding_mode_is_nearest()


def test_bf16_rne_against_library(orc):
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3e38)]
    ours = orc.bf16_rne(f)
    lib = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)
