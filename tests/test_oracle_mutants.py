"""Mutation tests of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of oracle/oracle.c: a wrong
exponent bias or mantissa weight, another rounding rule, a dropped term, a
transposed or shifted index, a missing sign.  The copy is built with the
oracle's own compiler flags into a temporary directory, the oracle's pin tests
(the four test_oracle_* files below) run against it in a subprocess, and at
least one pin must fail.  The oracle itself is never modified.

A mutant that no pin kills means the pins do not fix that part of the
definition; the test names the survivors.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = [os.path.join(ROOT, "tests", f) for f in
        ("test_oracle_codec.py", "test_oracle_quant.py", "test_oracle_gemm.py", "test_oracle_scale_fp32.py")]

# name: (text in oracle.c, which must occur exactly once; its replacement).
# Every replacement keeps all memory accesses inside the buffers.
MUTANTS = {
    # E4M3 decode
    "decode_exponent_bias_8": ("mag = ldexp(1.0 + m / 8.0, E - 7);", "mag = ldexp(1.0 + m / 8.0, E - 8);"),
    "decode_mantissa_weight": ("mag = ldexp(1.0 + m / 8.0, E - 7);", "mag = ldexp(1.0 + m / 16.0, E - 7);"),
    "decode_subnormal_step": ("mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    "decode_drops_sign": ("return sign ? -mag : mag;", "return mag;"),
    # E4M3 encode
    "encode_ties_away_from_zero": ("f = nearbyint((ldexp(a, -E) - 1.0) * 8.0);",
                                   "f = round((ldexp(a, -E) - 1.0) * 8.0);"),
    "encode_subnormal_truncates": ("double m = nearbyint(a * 512.0);", "double m = floor(a * 512.0);"),
    "encode_saturates_to_nan": ("        return sign | 0x7E;\n    if (a < ldexp(1.0, -6)) {",
                                "        return sign | 0x7F;\n    if (a < ldexp(1.0, -6)) {"),
    "encode_loses_negative_zero": ("    sign = signbit(v) ? 0x80 : 0x00;\n    a = fabs(v);",
                                   "    sign = v < 0 ? 0x80 : 0x00;\n    a = fabs(v);"),
    "encode_binade_carry_dropped": ("        E += 1;\n        f = 0.0;", "        f = 7.0;"),
    # bf16 output rounding
    "bf16_ties_away_from_zero": ("u += 0x7FFF + ((u >> 16) & 1);", "u += 0x8000;"),
    "bf16_truncates": ("u += 0x7FFF + ((u >> 16) & 1);", "u += 0;"),
    # power-of-two scale rule
    "scale_floor_rule": ("    while (amax <= ldexp(448.0, e - 1))\n        --e;\n",
                         "    while (amax <= ldexp(448.0, e - 1))\n        --e;\n"
                         "    if (amax < ldexp(448.0, e))\n        --e;\n"),
    "scale_one_too_large": ("    if (e < -126)\n        e = -126;", "    ++e;\n    if (e < -126)\n        e = -126;"),
    "scale_zero_group": ("    if (amax == 0.0)\n        return 0;", "    if (amax == 0.0)\n        return -126;"),
    "scale_clamp_127": ("    if (e < -126)\n        e = -126;", "    if (e < -127)\n        e = -127;"),
    # amax / 448 scale rule
    "fp32_scale_by_reciprocal": ("return amax / 448.0f;", "return amax * (1.0f / 448.0f);"),
    "fp32_scale_zero_group": ("    if (amax == 0.0f)\n        return 1.0f;", "    if (amax == 0.0f)\n        return 0.5f;"),
    "fp32_quotient_in_double": ("return orc_e4m3_encode((double)((float)x / s));",
                                "return orc_e4m3_encode(x / (double)s);"),
    # grouping
    "rowgroup_scale_transposed": ("s[r * G + g] = sc;", "s[g * rows + r] = sc;"),
    "rowgroup_amax_drops_last": ("            for (i = 0; i < GROUP; ++i) {\n"
                                 "                double v = fabs(orc_bf16_to_double(x[r * ld_x + g * GROUP + i]));",
                                 "            for (i = 0; i < GROUP - 1; ++i) {\n"
                                 "                double v = fabs(orc_bf16_to_double(x[r * ld_x + g * GROUP + i]));"),
    "rowgroup_ignores_ld_x": ("quantize_one(orc_bf16_to_double(x[r * ld_x + g * GROUP + i]), mode, e, sc);",
                              "quantize_one(orc_bf16_to_double(x[r * cols + g * GROUP + i]), mode, e, sc);"),
    "colgroup_codes_reversed": ("qT[c * ld_qT + g * GROUP + i] =", "qT[c * ld_qT + g * GROUP + (GROUP - 1 - i)] ="),
    "colgroup_amax_wrong_column": ("double v = fabs(orc_bf16_to_double(x[(g * GROUP + i) * ld_x + c]));",
                                   "double v = fabs(orc_bf16_to_double(x[(g * GROUP + i) * ld_x + (c ^ 1)]));"),
    "block_amax_half_columns": ("            for (c = bj * GROUP; c < (bj + 1) * GROUP; ++c) {\n                double v",
                                "            for (c = bj * GROUP; c < bj * GROUP + GROUP / 2; ++c) {\n"
                                "                double v"),
    "block_transpose_reversed": ("qT[c * rows + r] = code;", "qT[c * rows + (rows - 1 - r)] = code;"),
    "block_scale_transposed": ("s[bi * CB + bj] = sc;", "s[bj * RB + bi] = sc;"),
    # GEMMs
    "gemm_drops_b_scale": ("sc = (double)sa[kb * sa_step] * (double)sb[kb * sb_step];",
                           "sc = (double)sa[kb * sa_step];"),
    "gemm_drops_last_block": ("for (kb = 0; kb < R / GROUP; ++kb) {", "for (kb = 0; kb < R / GROUP - 1; ++kb) {"),
    "gemm_magnitudes_only": ("            p += t;", "            p += fabs(t);"),
    "gemm_sum_rounded_once": ("acc32 = acc32 + (float)(p * sc);", "acc32 = (float)(acc64 + p * sc);"),
    "fprop_weight_block_row": ("qw + n * K, 1, sw + (n / GROUP) * KB, 1,", "qw + n * K, 1, sw + (n / GROUP / 2) * KB, 1,"),
    "dgrad_scale_stride": ("qw + k, K, sw + k / GROUP, KB,", "qw + k, K, sw + k / GROUP, 1,"),
    "dgrad_weight_transposed": ("qw + k, K, sw + k / GROUP, KB,", "qw + k * N, 1, sw + k / GROUP, KB,"),
    "wgrad_x_scale_wrong_row": ("qxT + k * M, 1, sxT + k * MB, 1,", "qxT + k * M, 1, sxT + (k ^ 1) * MB, 1,"),
}


def _build(tmp, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"{name}: the text to mutate occurs {text.count(old)} times"
    src = os.path.join(tmp, f"{name}.c")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    import oracle
    so = os.path.join(tmp, f"{name}.so")
    subprocess.run(["gcc", *oracle._CFLAGS, "-o", so, src, "-lm"], check=True, capture_output=True)
    return so


def _killed(so):
    env = dict(os.environ, FP8BLK_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    if r.returncode not in (0, 1):
        # 1 is "some test failed"; anything else (a crash, a usage error) decides nothing
        raise RuntimeError(f"pin run ended with {r.returncode}:\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}")
    return r.returncode == 1


def test_every_mutant_is_killed_by_a_pin(tmp_path):
    if subprocess.run(["which", "gcc"], capture_output=True).returncode != 0:
        pytest.skip("no gcc")
    names = list(MUTANTS)
    with ThreadPoolExecutor(max_workers=6) as pool:
        killed = dict(zip(names, pool.map(lambda n: _killed(_build(str(tmp_path), n, *MUTANTS[n])), names)))
    survivors = [n for n, k in killed.items() if not k]
    assert not survivors, f"mutants no pin catches: {survivors}"


def test_unmutated_copy_passes_the_pins(tmp_path):
    """The harness itself: the oracle built the same way from the unchanged
    source passes every pin, so a kill above is the mutation's doing."""
    so = _build(str(tmp_path), "unchanged", "#define GROUP 128", "#define GROUP 128")
    assert not _killed(so)
