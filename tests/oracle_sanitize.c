/* Drives the oracle's entry points on small, exactly sized heap buffers so
 * that a build with address and undefined-behaviour sanitizers catches any
 * out-of-bounds access or undefined operation in oracle/oracle.c.  Test
 * infrastructure for tests/test_oracle_sanitize.py; it computes nothing of
 * its own beyond filling inputs. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double orc_e4m3_decode(uint8_t c);
uint8_t orc_e4m3_encode(double v);
uint8_t orc_e4m3_encode_nearest(double v);
uint16_t orc_bf16_rne(float f);
int orc_scale_exponent(double amax);
float orc_scale_fp32(float amax);
void orc_quantize_rowgroup(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *q, int64_t ld_q,
                           float *s, int mode);
void orc_quantize_colgroup(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *qT, int64_t ld_qT,
                           float *sT, int mode);
void orc_quantize_block(const uint16_t *w, int64_t rows, int64_t cols, int64_t ld_w, uint8_t *q, uint8_t *qT,
                        float *s, int mode);
void orc_gemm_fprop(int64_t M, int64_t N, int64_t K, const uint8_t *qx, const float *sx, const uint8_t *qw,
                    const float *sw, const int64_t *rows, int64_t nrows, float *y32, double *y64, double *bound);
void orc_gemm_dgrad(int64_t M, int64_t N, int64_t K, const uint8_t *qdy, const float *sdy, const uint8_t *qw,
                    const float *sw, const int64_t *rows, int64_t nrows, float *y32, double *y64, double *bound);
void orc_gemm_wgrad(int64_t M, int64_t N, int64_t K, const uint8_t *qdyT, const float *sdyT, const uint8_t *qxT,
                    const float *sxT, const int64_t *rows, int64_t nrows, float *y32, double *y64, double *bound);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(state >> 11) / 9007199254740992.0;
}

/* bf16 bits of rows x cols values (row stride ld), exactly the bytes a
 * strided tensor spans; a few all-zero groups, subnormals and large values */
static uint16_t *make_bf16(int64_t rows, int64_t cols, int64_t ld, double std)
{
    uint16_t *x = malloc(sizeof(uint16_t) * (size_t)((rows - 1) * ld + cols));
    int64_t r, c;
    for (r = 0; r < rows; ++r)
        for (c = 0; c < cols; ++c) {
            double u = uniform(), v = (2.0 * uniform() - 1.0) * std;
            if (u < 0.01) v *= 1e-38;          /* bf16 subnormal range */
            else if (u < 0.02) v *= 1e30;
            if (r == 1 && c < 128) v = 0.0;    /* an all-zero row group */
            x[r * ld + c] = orc_bf16_rne((float)v);
        }
    return x;
}

static int check_codes(const uint8_t *q, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        if ((q[i] & 0x7F) == 0x7F) return 1;   /* NaN code */
    return 0;
}

int main(void)
{
    int mode, bad = 0;
    for (mode = 0; mode < 2; ++mode) {
        /* row groups: ragged row count, strided input and output */
        {
            int64_t rows = 3, cols = 256, ld_x = 264, ld_q = 272;
            uint16_t *x = make_bf16(rows, cols, ld_x, 1.0);
            uint8_t *q = malloc((size_t)((rows - 1) * ld_q + cols));
            float *s = malloc(sizeof(float) * (size_t)(rows * (cols / 128)));
            orc_quantize_rowgroup(x, rows, cols, ld_x, q, ld_q, s, mode);
            bad |= check_codes(q, cols);
            free(x); free(q); free(s);
        }
        /* column groups, transposed output with a padded row stride */
        {
            int64_t rows = 256, cols = 384, ld_x = 392, ld_qT = 272;
            uint16_t *x = make_bf16(rows, cols, ld_x, 1.0);
            uint8_t *qT = malloc((size_t)((cols - 1) * ld_qT + rows));
            float *sT = malloc(sizeof(float) * (size_t)(cols * (rows / 128)));
            orc_quantize_colgroup(x, rows, cols, ld_x, qT, ld_qT, sT, mode);
            bad |= check_codes(qT, rows);
            free(x); free(qT); free(sT);
        }
        /* weight blocks, with and without the transposed copy */
        {
            int64_t rows = 256, cols = 384, ld_w = 400;
            uint16_t *w = make_bf16(rows, cols, ld_w, 0.02);
            uint8_t *q = malloc((size_t)(rows * cols)), *qT = malloc((size_t)(rows * cols));
            float *s = malloc(sizeof(float) * (size_t)((rows / 128) * (cols / 128)));
            orc_quantize_block(w, rows, cols, ld_w, q, qT, s, mode);
            orc_quantize_block(w, rows, cols, ld_w, q, NULL, s, mode);
            bad |= check_codes(q, rows * cols) | check_codes(qT, rows * cols);
            free(w); free(q); free(qT); free(s);
        }
    }
    /* the three GEMMs on row subsets, dense operands from the quantizers */
    {
        const int64_t M = 256, N = 384, K = 512;
        const int64_t rows_m[3] = {0, 5, M - 1}, rows_n[3] = {0, 130, N - 1};
        uint16_t *x = make_bf16(M, K, K, 1.0), *w = make_bf16(N, K, K, 0.02), *dy = make_bf16(M, N, N, 1e-3);
        uint8_t *qx = malloc((size_t)(M * K)), *qxT = malloc((size_t)(M * K)), *qw = malloc((size_t)(N * K));
        uint8_t *qdy = malloc((size_t)(M * N)), *qdyT = malloc((size_t)(M * N));
        float *sx = malloc(sizeof(float) * (size_t)(M * (K / 128))), *sxT = malloc(sizeof(float) * (size_t)(K * (M / 128)));
        float *sw = malloc(sizeof(float) * (size_t)((N / 128) * (K / 128)));
        float *sdy = malloc(sizeof(float) * (size_t)(M * (N / 128))), *sdyT = malloc(sizeof(float) * (size_t)(N * (M / 128)));
        float *y32 = malloc(sizeof(float) * (size_t)(3 * (N > K ? N : K)));
        double *y64 = malloc(sizeof(double) * (size_t)(3 * (N > K ? N : K)));
        double *bnd = malloc(sizeof(double) * (size_t)(3 * (N > K ? N : K)));
        orc_quantize_rowgroup(x, M, K, K, qx, K, sx, 0);
        orc_quantize_colgroup(x, M, K, K, qxT, M, sxT, 0);
        orc_quantize_block(w, N, K, K, qw, NULL, sw, 0);
        orc_quantize_rowgroup(dy, M, N, N, qdy, N, sdy, 0);
        orc_quantize_colgroup(dy, M, N, N, qdyT, M, sdyT, 0);
        orc_gemm_fprop(M, N, K, qx, sx, qw, sw, rows_m, 3, y32, y64, bnd);
        bad |= !isfinite(y64[3 * N - 1]);
        orc_gemm_dgrad(M, N, K, qdy, sdy, qw, sw, rows_m, 3, y32, y64, bnd);
        bad |= !isfinite(y64[3 * K - 1]);
        orc_gemm_wgrad(M, N, K, qdyT, sdyT, qxT, sxT, rows_n, 3, y32, y64, bnd);
        bad |= !isfinite(y64[3 * K - 1]);
        free(x); free(w); free(dy); free(qx); free(qxT); free(qw); free(qdy); free(qdyT);
        free(sx); free(sxT); free(sw); free(sdy); free(sdyT); free(y32); free(y64); free(bnd);
    }
    /* scalar helpers over their whole domains' edges */
    {
        int c;
        for (c = 0; c < 256; ++c) {
            double v = orc_e4m3_decode((uint8_t)c);
            if (!isnan(v)) bad |= orc_e4m3_encode(v) != c || orc_e4m3_encode_nearest(v) != c;
        }
        bad |= orc_scale_exponent(0.0) != 0 || orc_scale_fp32(0.0f) != 1.0f;
        (void)orc_scale_exponent(1e-45);
        (void)orc_scale_exponent(3.0e38);
        (void)orc_scale_fp32(3.0e38f);
        (void)orc_e4m3_encode(1e300);
        (void)orc_e4m3_encode(-1e-300);
    }
    printf("oracle sanitize run: %s\n", bad ? "FAILED checks" : "ok");
    return bad ? 1 : 0;
}
