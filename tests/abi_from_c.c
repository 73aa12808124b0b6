/*
 * The C ABI used from plain C99: include/fp8blk.h must compile as C, and
 * every entry point it declares must link against libfp8blk.so and reject
 * bad arguments with the documented status before it touches the device.
 *
 * Every call below carries at least one invalid argument, so none of them
 * reaches the device: the pointers are never dereferenced (non-null, 16-byte
 * aligned stand-ins) and the program needs no GPU.  Built and run by
 * tests/test_abi.py.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fp8blk.h"

static int failures = 0;

static void expect(const char *what, int got, int want)
{
    if (got != want) {
        printf("%s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

int main(void)
{
    /* stand-ins for device buffers: aligned, never dereferenced */
    uint16_t *x = (uint16_t *)(uintptr_t)0x100000;
    uint16_t *x_odd = (uint16_t *)(uintptr_t)0x100002;
    uint8_t *q = (uint8_t *)(uintptr_t)0x200000;
    uint8_t *qT = (uint8_t *)(uintptr_t)0x300000;
    float *s = (float *)(uintptr_t)0x400000;
    float *sT = (float *)(uintptr_t)0x500000;
    void *out = (void *)(uintptr_t)0x600000;
    void *out2 = (void *)(uintptr_t)0x700000;
    hipStream_t st = 0;
    fp8blk_block_job job;
    int codes[] = {FP8BLK_OK, FP8BLK_ERR_NULL, FP8BLK_ERR_DIM, FP8BLK_ERR_ALIGN, FP8BLK_ERR_ARG,
                   FP8BLK_ERR_WORKSPACE, FP8BLK_ERR_HIP, FP8BLK_ERR_DEVICE};
    size_t i, j;

    /* quantizers */
    expect("rowgroup null x", fp8_quantize_rowgroup(NULL, 128, 256, 256, q, 256, s, FP8BLK_SCALE_POW2, st),
           FP8BLK_ERR_NULL);
    expect("rowgroup ragged cols", fp8_quantize_rowgroup(x, 128, 200, 200, q, 200, s, FP8BLK_SCALE_POW2, st),
           FP8BLK_ERR_DIM);
    expect("rowgroup ld_x < cols", fp8_quantize_rowgroup(x, 128, 256, 128, q, 256, s, FP8BLK_SCALE_POW2, st),
           FP8BLK_ERR_ARG);
    expect("rowgroup misaligned x", fp8_quantize_rowgroup(x_odd, 128, 256, 256, q, 256, s, FP8BLK_SCALE_POW2, st),
           FP8BLK_ERR_ALIGN);
    expect("rowgroup scale mode", fp8_quantize_rowgroup(x, 128, 256, 256, q, 256, s, 7, st), FP8BLK_ERR_ARG);
    expect("colgroup ragged rows", fp8_quantize_colgroup(x, 200, 256, 256, qT, 200, sT, FP8BLK_SCALE_POW2, st),
           FP8BLK_ERR_DIM);
    expect("dual null qT", fp8_quantize_dual(x, 128, 256, 256, q, 256, s, NULL, 128, sT, FP8BLK_SCALE_FP32, st),
           FP8BLK_ERR_NULL);
    expect("block ld_w < cols", fp8_quantize_block(x, 256, 256, 128, q, NULL, s, FP8BLK_SCALE_POW2, st),
           FP8BLK_ERR_ARG);
    job.w = x;
    job.rows = 0;
    job.cols = 256;
    job.ld_w = 256;
    job.q = q;
    job.qT = NULL;
    job.s = s;
    expect("block batch no jobs", fp8_quantize_block_batch(&job, 0, FP8BLK_SCALE_POW2, st), FP8BLK_ERR_ARG);
    expect("block batch null jobs", fp8_quantize_block_batch(NULL, 1, FP8BLK_SCALE_POW2, st), FP8BLK_ERR_NULL);
    expect("block batch empty job", fp8_quantize_block_batch(&job, 1, FP8BLK_SCALE_POW2, st), FP8BLK_ERR_DIM);

    /* GEMMs */
    expect("fprop M = 0", fp8_block_gemm_fprop(0, 256, 256, q, s, qT, sT, out, FP8BLK_OUT_BF16, st), FP8BLK_ERR_DIM);
    expect("fprop out dtype", fp8_block_gemm_fprop(256, 256, 256, q, s, qT, sT, out, 9, st), FP8BLK_ERR_ARG);
    expect("dgrad null sw", fp8_block_gemm_dgrad(256, 256, 256, q, s, qT, NULL, out, FP8BLK_OUT_BF16, st),
           FP8BLK_ERR_NULL);
    expect("dgrad_w ragged K", fp8_block_gemm_dgrad_w(256, 256, 200, q, s, qT, sT, out, FP8BLK_OUT_BF16, st),
           FP8BLK_ERR_DIM);
    /* the O projection's Wgrad shares tiles among workgroups: it needs a workspace */
    expect("wgrad no workspace",
           fp8_block_gemm_wgrad(8192, 2048, 2048, qT, sT, q, s, out, FP8BLK_OUT_BF16, NULL, 0, st),
           FP8BLK_ERR_WORKSPACE);
    expect("backward dx == dw",
           fp8_block_gemm_backward(256, 256, 256, q, s, qT, sT, qT, sT, q, s, out, FP8BLK_OUT_BF16, out,
                                   FP8BLK_OUT_BF16, FP8BLK_SCALE_POW2, NULL, 0, st),
           FP8BLK_ERR_ARG);
    expect("backward_w misaligned dY codes",
           fp8_block_gemm_backward_w(256, 256, 256, q + 1, s, qT, sT, qT, sT, q, s, out, FP8BLK_OUT_BF16, out2,
                                     FP8BLK_OUT_FP32, FP8BLK_SCALE_POW2, NULL, 0, st),
           FP8BLK_ERR_ALIGN);
    expect("gemm bad op", fp8_block_gemm(9, 256, 256, 256, q, s, qT, sT, out, FP8BLK_OUT_BF16, FP8BLK_ALGO_DEFAULT,
                                         FP8BLK_SCALE_POW2, NULL, 0, st),
           FP8BLK_ERR_ARG);
    expect("gemm bad algo", fp8_block_gemm(FP8BLK_OP_FPROP, 256, 256, 256, q, s, qT, sT, out, FP8BLK_OUT_BF16, 5,
                                           FP8BLK_SCALE_POW2, NULL, 0, st),
           FP8BLK_ERR_ARG);
    /* amax / 448 scales keep their mantissa only in the promote algorithm */
    expect("gemm fp32 scales, scaled MFMA",
           fp8_block_gemm(FP8BLK_OP_FPROP, 256, 256, 256, q, s, qT, sT, out, FP8BLK_OUT_BF16,
                          FP8BLK_ALGO_SCALED_MFMA, FP8BLK_SCALE_FP32, NULL, 0, st),
           FP8BLK_ERR_ARG);
    expect("gemm bad scale mode",
           fp8_block_gemm(FP8BLK_OP_FPROP, 256, 256, 256, q, s, qT, sT, out, FP8BLK_OUT_BF16, FP8BLK_ALGO_DEFAULT,
                          2, NULL, 0, st),
           FP8BLK_ERR_ARG);
    expect("backward bad scale mode",
           fp8_block_gemm_backward_w(256, 256, 256, q, s, qT, sT, qT, sT, q, s, out, FP8BLK_OUT_BF16, out2,
                                     FP8BLK_OUT_FP32, -1, NULL, 0, st),
           FP8BLK_ERR_ARG);

    /* helpers */
    expect("workspace fprop", (int)fp8_block_gemm_workspace_size(FP8BLK_OP_FPROP, 8192, 12288, 2048), 0);
    expect("workspace bad op", fp8_block_gemm_workspace_size(9, 256, 256, 256) == (size_t)-1, 1);
    expect("workspace O wgrad", fp8_block_gemm_workspace_size(FP8BLK_OP_WGRAD, 8192, 2048, 2048) > 0, 1);
    for (i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
        const char *a = fp8_status_string(codes[i]);
        expect("status string present", a != NULL && a[0] != '\0', 1);
        for (j = 0; j < i; ++j)
            expect("status strings distinct", strcmp(a, fp8_status_string(codes[j])) != 0, 1);
    }

    if (failures == 0)
        printf("ok\n");
    return failures == 0 ? 0 : 1;
}
