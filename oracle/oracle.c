/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the blockwise-FP8
 * Transformer linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library; it is written from the method's definition.
 *
 * Sources ("the pages"):
 *   [P1]  "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090"
 *         (arXiv HTML, part 3/7), section 3.2 "FP8 Mixed-Precision Training".
 *   [P3]  Chinese study notes of the same paper (arXiv v2), section 2.3
 *         (the FP8 boundary table).
 *   [P5]  "Tsinghua's PuRo-2B trains from scratch on RTX 5090s ..." (paper
 *         explainer), section "Method", FP8 bullet.
 *   [OCP] Micikevicius et al. 2022, "FP8 Formats for Deep Learning", Table 1
 *         (the E4M3 definition that [P1] section 3.2 cites).
 *
 * What is computed (readings where the pages are silent are marked READING):
 *   - E4M3 operands [P1 s3.2 para 1; P3 s2.3 table], OCP "fn" variant [OCP
 *     Table 1]: bias 7, no infinities, S.1111.111 is NaN, max 448.
 *   - activations / gradients: a scale for every 128-element group taken
 *     along K, the contracted dimension [P1 s3.2 para 2; P3 s2.3 table;
 *     P5 Method];
 *     weights: one scale per 128x128 block [same places].
 *   - every scale is a power of two (E8M0-like) [P1 s3.2 para 3; P3 s2.3].
 *     READING: s = 2^e with e the smallest integer such that amax <= 448*2^e
 *     (no value of the group is clipped), e clamped to [-126, 127]; an
 *     all-zero group has s = 1.  s is stored as an fp32 multiplier (x ~ q*s).
 *   - q = RNE-to-E4M3(x / s), saturating at +-448; the division by a power of
 *     two is exact, so there is a single rounding.
 *   - mode 1, a numerics variant (FP8BLK_SCALE_FP32): [P1 s3.2 para 3] sets
 *     the run's power-of-two scale against the DeepSeek-V3 recipe it follows
 *     otherwise, without printing that recipe's formula.  READING: the scale
 *     that puts the group's amax on 448 exactly, s = fl32(amax / 448) (IEEE
 *     single division; amax is a bf16 value, exact in float), s = 1 for an
 *     all-zero group, and q = RNE-to-E4M3(fl32(x / s)) saturating at +-448
 *     (the rounded quotient of the amax itself can exceed 448 by an ulp).
 *   - GEMMs (Fprop, Dgrad, Wgrad all on the FP8 path [P1 s3.2 para 4; P3 s2.3]):
 *     out[i][j] = sum over 128-deep reduction blocks b of
 *                 sa(i,b) * sb(j,b) * sum_{r in b} dec(A[i][r]) * dec(B[j][r]).
 *     Three results are produced per output element:
 *       y64   : the sum above in double (the per-block inner sum of E4M3
 *               products is exact in double: every product is a multiple of
 *               2^-18 below 2^18, 128 of them need < 44 bits);
 *       y32   : READING of "fp32 accumulation": each exact block term
 *               p*sa*sb is rounded once to fp32 and added to an fp32
 *               accumulator in increasing block order (with mode-1 scales,
 *               which are not powers of two, the term is first formed in
 *               double: one extra rounding of 2^-53, far inside every
 *               tolerance that y32 serves);
 *       bound : sum over all terms of |sa*dec*sb*dec| (double), the scale that
 *               any summation-order error is proportional to.
 *   - bf16 output: round-to-nearest-even of the fp32 result [P1 s3.2 para 4:
 *     BF16 output materialised for the surrounding model].
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off (no fast-math).
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GROUP 128

/* ---------------------------------------------------------------- E4M3 --- */

/* [OCP Table 1]: sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal: m * 2^-9.  Otherwise (1 + m/8) * 2^(E-7).
 * S.1111.111 is NaN; there is no infinity. */
double orc_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int E = (c >> 3) & 15;
    int m = c & 7;
    double mag;
    if (E == 15 && m == 7)
        return NAN;
    if (E == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, E - 7);
    return sign ? -mag : mag;
}

/* Encoder 1 -- by arithmetic.  Round to nearest, ties to even, saturating
 * at the largest finite magnitude 448 (code 0x7E).  Sign is kept (-0 -> 0x80).
 * NaN inputs are outside the contract and map to 0x7F. */
uint8_t orc_e4m3_encode(double v)
{
    uint8_t sign;
    double a, f;
    int E, code;
    if (isnan(v))
        return 0x7F;
    sign = signbit(v) ? 0x80 : 0x00;
    a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: grid step 2^-9; m == 8 lands on the smallest
         * normal, whose code is 0x08, so the integer is the code itself */
        double m = nearbyint(a * 512.0);
        return sign | (uint8_t)m;
    }
    frexp(a, &E);
    E -= 1;                                /* a = (1.f) * 2^E */
    f = nearbyint((ldexp(a, -E) - 1.0) * 8.0);
    if (f == 8.0) {                        /* rounded up into the next binade */
        E += 1;
        f = 0.0;
    }
    code = ((E + 7) << 3) | (int)f;
    if (code > 0x7E)                       /* unreachable for a < 448 */
        code = 0x7E;
    return sign | (uint8_t)code;
}

/* Encoder 2 -- by search: the nearest of the 127 non-negative finite codes to
 * min(|v|, 448), ties to the code whose last bit is 0.  Independent of the
 * arithmetic above; the two must agree everywhere. */
uint8_t orc_e4m3_encode_nearest(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v), bestd = INFINITY;
    int c, best = 0;
    if (a > 448.0)
        a = 448.0;
    for (c = 0; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3_decode((uint8_t)c) - a);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            bestd = d;
            best = c;
        }
    }
    return sign | (uint8_t)best;
}

/* ---------------------------------------------------------------- bf16 --- */

double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* fp32 -> bf16, round to nearest even (finite inputs). */
uint16_t orc_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return 0x7FC0;
    u += 0x7FFF + ((u >> 16) & 1);
    return (uint16_t)(u >> 16);
}

/* --------------------------------------------------------------- scales --- */

/* READING of the power-of-two scale [P1 s3.2 para 3]: the smallest integer e
 * with amax <= 448 * 2^e, clamped to [-126, 127]; 0 for an all-zero group. */
int orc_scale_exponent(double amax)
{
    int e;
    if (amax == 0.0)
        return 0;
    frexp(amax / 448.0, &e);               /* a starting guess only */
    while (amax > ldexp(448.0, e))
        ++e;
    while (amax <= ldexp(448.0, e - 1))
        --e;
    if (e < -126)
        e = -126;
    if (e > 127)
        e = 127;
    return e;
}

/* READING of the mode-1 scale (see the header): fl32(amax / 448), 1 for 0. */
float orc_scale_fp32(float amax)
{
    if (amax == 0.0f)
        return 1.0f;
    return amax / 448.0f;
}

/* The scale of a group with this amax under `mode`; for mode 0 also its
 * exponent e (s = 2^e). */
static float group_scale(double amax, int mode, int *e)
{
    if (mode == 0) {
        *e = orc_scale_exponent(amax);
        return ldexpf(1.0f, *e);
    }
    *e = 0;
    return orc_scale_fp32((float)amax);
}

/* The code of element x of a group: mode 0 encodes the exact x * 2^-e,
 * mode 1 the single-precision quotient fl32(x / s). */
static uint8_t quantize_one(double x, int mode, int e, float s)
{
    if (mode == 0)
        return orc_e4m3_encode(ldexp(x, -e));
    return orc_e4m3_encode((double)((float)x / s));
}

/* ----------------------------------------------------------- quantizers --- */

/* Row groups [P1 s3.2 para 2]: x is rows x cols (row stride ld_x), groups are
 * 128 consecutive elements of a row.  q is rows x cols (row stride ld_q),
 * s is rows x (cols/128), dense.  mode: the scale rule (0 power of two,
 * 1 amax / 448), as for the other two quantizers. */
void orc_quantize_rowgroup(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t *q, int64_t ld_q, float *s, int mode)
{
    int64_t G = cols / GROUP;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        int64_t g;
        for (g = 0; g < G; ++g) {
            double amax = 0.0;
            float sc;
            int i, e;
            for (i = 0; i < GROUP; ++i) {
                double v = fabs(orc_bf16_to_double(x[r * ld_x + g * GROUP + i]));
                if (v > amax)
                    amax = v;
            }
            sc = group_scale(amax, mode, &e);
            s[r * G + g] = sc;
            for (i = 0; i < GROUP; ++i)
                q[r * ld_q + g * GROUP + i] =
                    quantize_one(orc_bf16_to_double(x[r * ld_x + g * GROUP + i]), mode, e, sc);
        }
    }
}

/* Column groups: the same rule with groups of 128 consecutive ROWS of one
 * column (the token dimension, which is Wgrad's reduction dimension), written
 * transposed: qT is cols x rows (row stride ld_qT), sT is cols x (rows/128). */
void orc_quantize_colgroup(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t *qT, int64_t ld_qT, float *sT, int mode)
{
    int64_t G = rows / GROUP;
    int64_t c;
#pragma omp parallel for schedule(static)
    for (c = 0; c < cols; ++c) {
        int64_t g;
        for (g = 0; g < G; ++g) {
            double amax = 0.0;
            float sc;
            int i, e;
            for (i = 0; i < GROUP; ++i) {
                double v = fabs(orc_bf16_to_double(x[(g * GROUP + i) * ld_x + c]));
                if (v > amax)
                    amax = v;
            }
            sc = group_scale(amax, mode, &e);
            sT[c * G + g] = sc;
            for (i = 0; i < GROUP; ++i)
                qT[c * ld_qT + g * GROUP + i] =
                    quantize_one(orc_bf16_to_double(x[(g * GROUP + i) * ld_x + c]), mode, e, sc);
        }
    }
}

/* 128x128 blocks [P1 s3.2 para 2]: w is rows x cols (row stride ld_w); q is
 * rows x cols dense; qT (optional, may be NULL) is cols x rows dense; s is
 * (rows/128) x (cols/128). */
void orc_quantize_block(const uint16_t *w, int64_t rows, int64_t cols, int64_t ld_w,
                        uint8_t *q, uint8_t *qT, float *s, int mode)
{
    int64_t RB = rows / GROUP, CB = cols / GROUP;
    int64_t blk;
#pragma omp parallel for schedule(static)
    for (blk = 0; blk < RB * CB; ++blk) {
        int64_t bi = blk / CB, bj = blk % CB, r, c;
        double amax = 0.0;
        float sc;
        int e;
        for (r = bi * GROUP; r < (bi + 1) * GROUP; ++r)
            for (c = bj * GROUP; c < (bj + 1) * GROUP; ++c) {
                double v = fabs(orc_bf16_to_double(w[r * ld_w + c]));
                if (v > amax)
                    amax = v;
            }
        sc = group_scale(amax, mode, &e);
        s[bi * CB + bj] = sc;
        for (r = bi * GROUP; r < (bi + 1) * GROUP; ++r)
            for (c = bj * GROUP; c < (bj + 1) * GROUP; ++c) {
                uint8_t code = quantize_one(orc_bf16_to_double(w[r * ld_w + c]), mode, e, sc);
                q[r * cols + c] = code;
                if (qT)
                    qT[c * rows + r] = code;
            }
    }
}

/* ---------------------------------------------------------------- GEMMs --- */

/* One output element: sum over reduction blocks of sa*sb*(exact inner sum).
 * a[r] is read at a + r*a_step, b[r] at b + r*b_step; the scales of block kb
 * at sa[kb*sa_step] and sb[kb*sb_step]. */
static void dot_blockscaled(int64_t R,
                            const uint8_t *a, int64_t a_step, const float *sa, int64_t sa_step,
                            const uint8_t *b, int64_t b_step, const float *sb, int64_t sb_step,
                            float *y32, double *y64, double *bound)
{
    float acc32 = 0.0f;
    double acc64 = 0.0, bnd = 0.0;
    int64_t kb, r;
    for (kb = 0; kb < R / GROUP; ++kb) {
        double p = 0.0, pabs = 0.0, sc;
        for (r = kb * GROUP; r < (kb + 1) * GROUP; ++r) {
            double t = orc_e4m3_decode(a[r * a_step]) * orc_e4m3_decode(b[r * b_step]);
            p += t;
            pabs += fabs(t);
        }
        sc = (double)sa[kb * sa_step] * (double)sb[kb * sb_step];
        acc32 = acc32 + (float)(p * sc);
        acc64 += p * sc;
        bnd += pabs * sc;
    }
    *y32 = acc32;
    *y64 = acc64;
    *bound = bnd;
}

/* Fprop  Y = X W^T  [P1 s3.2 para 4]:  Y[m][n] over k, X row-grouped along K,
 * W in 128x128 blocks.  qx: M x K, sx: M x K/128, qw: N x K, sw: N/128 x K/128.
 * Computes the listed rows m = rows[t]; outputs are nrows x N. */
void orc_gemm_fprop(int64_t M, int64_t N, int64_t K,
                    const uint8_t *qx, const float *sx, const uint8_t *qw, const float *sw,
                    const int64_t *rows, int64_t nrows, float *y32, double *y64, double *bound)
{
    int64_t KB = K / GROUP, t;
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < nrows; ++t) {
        int64_t m = rows[t], n;
        for (n = 0; n < N; ++n)
            dot_blockscaled(K, qx + m * K, 1, sx + m * KB, 1,
                            qw + n * K, 1, sw + (n / GROUP) * KB, 1,
                            y32 + t * N + n, y64 + t * N + n, bound + t * N + n);
    }
}

/* Dgrad  dX = dY W:  dX[m][k] over n, dY row-grouped along N, W the same
 * 128x128 blocks as Fprop, read directly as W[n][k] (no transposed copy).
 * qdy: M x N, sdy: M x N/128, qw: N x K, sw: N/128 x K/128.  Outputs nrows x K. */
void orc_gemm_dgrad(int64_t M, int64_t N, int64_t K,
                    const uint8_t *qdy, const float *sdy, const uint8_t *qw, const float *sw,
                    const int64_t *rows, int64_t nrows, float *y32, double *y64, double *bound)
{
    int64_t NB = N / GROUP, KB = K / GROUP, t;
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < nrows; ++t) {
        int64_t m = rows[t], k;
        for (k = 0; k < K; ++k)
            dot_blockscaled(N, qdy + m * N, 1, sdy + m * NB, 1,
                            qw + k, K, sw + k / GROUP, KB,
                            y32 + t * K + k, y64 + t * K + k, bound + t * K + k);
    }
}

/* Wgrad  dW = dY^T X:  dW[n][k] over m (tokens).  Both operands are grouped
 * along the token dimension, i.e. they are the column-group quantizations,
 * stored transposed: qdyT: N x M, sdyT: N x M/128, qxT: K x M, sxT: K x M/128.
 * Computes the listed output rows n = rows[t]; outputs are nrows x K. */
void orc_gemm_wgrad(int64_t M, int64_t N, int64_t K,
                    const uint8_t *qdyT, const float *sdyT, const uint8_t *qxT, const float *sxT,
                    const int64_t *rows, int64_t nrows, float *y32, double *y64, double *bound)
{
    int64_t MB = M / GROUP, t;
    (void)N;
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < nrows; ++t) {
        int64_t n = rows[t], k;
        for (k = 0; k < K; ++k)
            dot_blockscaled(M, qdyT + n * M, 1, sdyT + n * MB, 1,
                            qxT + k * M, 1, sxT + k * MB, 1,
                            y32 + t * K + k, y64 + t * K + k, bound + t * K + k);
    }
}

/* Vectorised helpers for the tests. */
void orc_e4m3_encode_array(const double *v, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(v[i]);
}

void orc_e4m3_encode_nearest_array(const double *v, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode_nearest(v[i]);
}

void orc_bf16_rne_array(const float *v, int64_t n, uint16_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = orc_bf16_rne(v[i]);
}

int orc_rounding_mode_is_nearest(void)
{
    return fegetround() == FE_TONEAREST;
}
