/*
 * GPU parity through the C ABI alone, from plain C99: no Python, no torch.
 * Device memory comes from hipMalloc, inputs from a seeded generator below,
 * and every result is checked against the CPU oracle (oracle/liboracle.so,
 * linked in as the reference):
 *   - codes and scales of the row-group, column-group, one-pass and block
 *     quantizers bit for bit;
 *   - Fprop, Dgrad (from the transposed codes and from the codes as
 *     quantized), Wgrad and the fused backward within the GEMM tolerance:
 *     |y - y32| <= 1e-3 * bound per element and 1e-3 * max|y32| overall for
 *     fp32 outputs, plus half a bf16 ulp of |y32| for bf16 outputs.
 * Shapes are multiples of 128 that leave partial 256 x 256 output tiles.
 * Built by __graft_entry__.build(); run by tests/test_gpu_c_abi.py.
 * Prints "ok" and exits 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fp8blk.h"

/* the oracle's entry points (oracle/oracle.c) */
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

enum { M = 384, N = 640, K = 512 };

static int failures = 0;

#define HIP(call)                                                                   \
    do {                                                                            \
        hipError_t e_ = (call);                                                     \
        if (e_ != hipSuccess) {                                                     \
            printf("%s:%d %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
            exit(2);                                                                \
        }                                                                           \
    } while (0)

#define FP8(call)                                                                   \
    do {                                                                            \
        int rc_ = (call);                                                           \
        if (rc_ != FP8BLK_OK) {                                                     \
            printf("%s:%d %s: %s\n", __FILE__, __LINE__, #call, fp8_status_string(rc_)); \
            exit(2);                                                                \
        }                                                                           \
    } while (0)

/* splitmix64: seeded input generation only */
static uint64_t rng_state;
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* bf16 bits of a value of random sign, magnitude spread over 2^lo .. 2^hi */
static uint16_t random_bf16(int lo, int hi)
{
    uint64_t r = next_u64();
    float f = ldexpf(1.0f + (float)(r & 0xFFFF) / 65536.0f, lo + (int)((r >> 16) % (uint64_t)(hi - lo + 1)));
    uint32_t u;
    if (r >> 63)
        f = -f;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static void *dev_alloc(size_t bytes)
{
    void *p = NULL;
    HIP(hipMalloc(&p, bytes));
    return p;
}

static void *to_host(const void *d, size_t bytes)
{
    void *h = malloc(bytes);
    if (!h) {
        printf("out of host memory\n");
        exit(2);
    }
    HIP(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    return h;
}

static void same_bytes(const char *what, const void *dev, const void *ref, size_t bytes)
{
    void *h = to_host(dev, bytes);
    if (memcmp(h, ref, bytes) != 0) {
        printf("%s: differs from the oracle\n", what);
        ++failures;
    }
    free(h);
}

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* a rows x cols GEMM output on the device (fp32 or bf16) against the
 * oracle's y32 and bound for the same elements */
static void within_tolerance(const char *what, const void *dev, int bf16, int64_t rows, int64_t cols,
                             const float *y32, const double *bound)
{
    size_t n = (size_t)(rows * cols), i;
    void *h = to_host(dev, n * (bf16 ? 2 : 4));
    double worst = 0.0, ymax = 0.0;
    int bad = 0;
    for (i = 0; i < n; ++i) {
        double y = bf16 ? bf16_to_float(((uint16_t *)h)[i]) : ((float *)h)[i];
        double err = fabs(y - (double)y32[i]);
        /* bf16: the rounding of the kernel's fp32 value adds at most half an
         * ulp, 2^-8 of that value's magnitude */
        double allowed = 1e-3 * bound[i] * (bf16 ? 1.0 + ldexp(1.0, -8) : 1.0) +
                         (bf16 ? ldexp(fabs((double)y32[i]), -8) : 0.0);
        if (!(err <= allowed))
            ++bad;
        if (!bf16 && err > worst)
            worst = err;
        if (fabs((double)y32[i]) > ymax)
            ymax = fabs((double)y32[i]);
    }
    if (bad || worst > 1e-3 * ymax) {
        printf("%s: %d elements outside the tolerance, normwise %.3g\n", what, bad, ymax > 0 ? worst / ymax : worst);
        ++failures;
    }
    free(h);
}

int main(void)
{
    int dev = 0, i;
    hipDeviceProp_t prop;
    HIP(hipGetDevice(&dev));
    HIP(hipGetDeviceProperties(&prop, dev));
    printf("device %d: %s\n", dev, prop.gcnArchName);

    /* ---- inputs: X [M][K], W [N][K], dY [M][N]; the first group of X's
     * row 5 is all zero, one of W's blocks holds an outlier */
    rng_state = 2024;
    uint16_t *x = malloc(sizeof(uint16_t) * M * K), *w = malloc(sizeof(uint16_t) * N * K),
             *dy = malloc(sizeof(uint16_t) * M * N);
    for (i = 0; i < M * K; ++i)
        x[i] = random_bf16(-6, 2);
    for (i = 0; i < N * K; ++i)
        w[i] = random_bf16(-12, -5);
    for (i = 0; i < M * N; ++i)
        dy[i] = random_bf16(-14, -8);
    memset(x + 5 * K, 0, 128 * sizeof(uint16_t));
    w[3 * K + 200] = 0x4300; /* 128.0 */

    uint16_t *d_x = dev_alloc(sizeof(uint16_t) * M * K), *d_w = dev_alloc(sizeof(uint16_t) * N * K),
             *d_dy = dev_alloc(sizeof(uint16_t) * M * N);
    HIP(hipMemcpy(d_x, x, sizeof(uint16_t) * M * K, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_w, w, sizeof(uint16_t) * N * K, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_dy, dy, sizeof(uint16_t) * M * N, hipMemcpyHostToDevice));

    /* ---- the oracle's quantizations */
    uint8_t *ox = malloc(M * K), *oxT = malloc(M * K), *ow = malloc(N * K), *owT = malloc(N * K),
            *ody = malloc(M * N), *odyT = malloc(M * N);
    float *osx = malloc(sizeof(float) * M * (K / 128)), *osxT = malloc(sizeof(float) * K * (M / 128)),
          *osw = malloc(sizeof(float) * (N / 128) * (K / 128)), *osdy = malloc(sizeof(float) * M * (N / 128)),
          *osdyT = malloc(sizeof(float) * N * (M / 128));
    orc_quantize_rowgroup(x, M, K, K, ox, K, osx, 0);
    orc_quantize_colgroup(x, M, K, K, oxT, M, osxT, 0);
    orc_quantize_block(w, N, K, K, ow, owT, osw, 0);
    orc_quantize_rowgroup(dy, M, N, N, ody, N, osdy, 0);
    orc_quantize_colgroup(dy, M, N, N, odyT, M, osdyT, 0);

    /* ---- the library's quantizations */
    uint8_t *qx = dev_alloc(M * K), *qxT = dev_alloc(M * K), *qx2 = dev_alloc(M * K), *qxT2 = dev_alloc(M * K),
            *qw = dev_alloc(N * K), *qwT = dev_alloc(N * K), *qdy = dev_alloc(M * N), *qdyT = dev_alloc(M * N);
    float *sx = dev_alloc(sizeof(float) * M * (K / 128)), *sxT = dev_alloc(sizeof(float) * K * (M / 128)),
          *sx2 = dev_alloc(sizeof(float) * M * (K / 128)), *sxT2 = dev_alloc(sizeof(float) * K * (M / 128)),
          *sw = dev_alloc(sizeof(float) * (N / 128) * (K / 128)), *sdy = dev_alloc(sizeof(float) * M * (N / 128)),
          *sdyT = dev_alloc(sizeof(float) * N * (M / 128));
    FP8(fp8_quantize_rowgroup(d_x, M, K, K, qx, K, sx, FP8BLK_SCALE_POW2, 0));
    FP8(fp8_quantize_colgroup(d_x, M, K, K, qxT, M, sxT, FP8BLK_SCALE_POW2, 0));
    FP8(fp8_quantize_dual(d_x, M, K, K, qx2, K, sx2, qxT2, M, sxT2, FP8BLK_SCALE_POW2, 0));
    FP8(fp8_quantize_block(d_w, N, K, K, qw, qwT, sw, FP8BLK_SCALE_POW2, 0));
    FP8(fp8_quantize_dual(d_dy, M, N, N, qdy, N, sdy, qdyT, M, sdyT, FP8BLK_SCALE_POW2, 0));
    HIP(hipDeviceSynchronize());
    same_bytes("X row-group codes", qx, ox, M * K);
    same_bytes("X row-group scales", sx, osx, sizeof(float) * M * (K / 128));
    same_bytes("X column-group codes", qxT, oxT, M * K);
    same_bytes("X column-group scales", sxT, osxT, sizeof(float) * K * (M / 128));
    same_bytes("X one-pass row codes", qx2, ox, M * K);
    same_bytes("X one-pass row scales", sx2, osx, sizeof(float) * M * (K / 128));
    same_bytes("X one-pass column codes", qxT2, oxT, M * K);
    same_bytes("X one-pass column scales", sxT2, osxT, sizeof(float) * K * (M / 128));
    same_bytes("W block codes", qw, ow, N * K);
    same_bytes("W transposed block codes", qwT, owT, N * K);
    same_bytes("W block scales", sw, osw, sizeof(float) * (N / 128) * (K / 128));
    same_bytes("dY one-pass row codes", qdy, ody, M * N);
    same_bytes("dY one-pass row scales", sdy, osdy, sizeof(float) * M * (N / 128));
    same_bytes("dY one-pass column codes", qdyT, odyT, M * N);
    same_bytes("dY one-pass column scales", sdyT, osdyT, sizeof(float) * N * (M / 128));

    /* ---- the oracle's GEMMs, every output row */
    int64_t *rows = malloc(sizeof(int64_t) * (M > N ? M : N));
    for (i = 0; i < (M > N ? M : N); ++i)
        rows[i] = i;
    float *y32 = malloc(sizeof(float) * M * N), *dx32 = malloc(sizeof(float) * M * K),
          *dw32 = malloc(sizeof(float) * N * K);
    double *y64 = malloc(sizeof(double) * M * N), *yb = malloc(sizeof(double) * M * N),
           *dx64 = malloc(sizeof(double) * M * K), *dxb = malloc(sizeof(double) * M * K),
           *dw64 = malloc(sizeof(double) * N * K), *dwb = malloc(sizeof(double) * N * K);
    orc_gemm_fprop(M, N, K, ox, osx, ow, osw, rows, M, y32, y64, yb);
    orc_gemm_dgrad(M, N, K, ody, osdy, ow, osw, rows, M, dx32, dx64, dxb);
    orc_gemm_wgrad(M, N, K, odyT, osdyT, oxT, osxT, rows, N, dw32, dw64, dwb);

    /* ---- the library's GEMMs */
    void *y = dev_alloc(sizeof(float) * M * N), *yh = dev_alloc(sizeof(uint16_t) * M * N),
         *dx = dev_alloc(sizeof(float) * M * K), *dxh = dev_alloc(sizeof(uint16_t) * M * K),
         *dw = dev_alloc(sizeof(float) * N * K), *dwh = dev_alloc(sizeof(uint16_t) * N * K),
         *dx2 = dev_alloc(sizeof(float) * M * K), *dw2 = dev_alloc(sizeof(float) * N * K);
    size_t ws_w = fp8_block_gemm_workspace_size(FP8BLK_OP_WGRAD, M, N, K);
    size_t ws_b = fp8_block_gemm_workspace_size(FP8BLK_OP_BACKWARD, M, N, K);
    size_t ws_bytes = (ws_w > ws_b ? ws_w : ws_b) + 16;
    void *ws = dev_alloc(ws_bytes);
    FP8(fp8_block_gemm_fprop(M, N, K, qx, sx, qw, sw, y, FP8BLK_OUT_FP32, 0));
    FP8(fp8_block_gemm_fprop(M, N, K, qx, sx, qw, sw, yh, FP8BLK_OUT_BF16, 0));
    FP8(fp8_block_gemm_dgrad(M, N, K, qdy, sdy, qwT, sw, dx, FP8BLK_OUT_FP32, 0));
    FP8(fp8_block_gemm_dgrad_w(M, N, K, qdy, sdy, qw, sw, dxh, FP8BLK_OUT_BF16, 0));
    FP8(fp8_block_gemm_wgrad(M, N, K, qdyT, sdyT, qxT, sxT, dw, FP8BLK_OUT_FP32, ws, ws_bytes, 0));
    FP8(fp8_block_gemm_wgrad(M, N, K, qdyT, sdyT, qxT, sxT, dwh, FP8BLK_OUT_BF16, ws, ws_bytes, 0));
    FP8(fp8_block_gemm_backward_w(M, N, K, qdy, sdy, qw, sw, qdyT, sdyT, qxT, sxT, dx2, FP8BLK_OUT_FP32, dw2,
                                  FP8BLK_OUT_FP32, FP8BLK_SCALE_POW2, ws, ws_bytes, 0));
    HIP(hipDeviceSynchronize());
    within_tolerance("fprop fp32", y, 0, M, N, y32, yb);
    within_tolerance("fprop bf16", yh, 1, M, N, y32, yb);
    within_tolerance("dgrad fp32", dx, 0, M, K, dx32, dxb);
    within_tolerance("dgrad_w bf16", dxh, 1, M, K, dx32, dxb);
    within_tolerance("wgrad fp32", dw, 0, N, K, dw32, dwb);
    within_tolerance("wgrad bf16", dwh, 1, N, K, dw32, dwb);
    within_tolerance("backward_w dx fp32", dx2, 0, M, K, dx32, dxb);
    within_tolerance("backward_w dw fp32", dw2, 0, N, K, dw32, dwb);

    if (failures == 0)
        printf("ok\n");
    return failures == 0 ? 0 : 1;
}
