/*
 * fp8blk.h -- C ABI of the blockwise-FP8 Transformer linear layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (sources, cited by title and section):
 *   "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090"
 *   (arXiv HTML, part 3/7), section 3.2 "FP8 Mixed-Precision Training":
 *     - Transformer linear layers take E4M3 operands; the BF16 inputs and
 *       weights are quantized right before each GEMM and a BF16 output is
 *       materialised (fourth paragraph);
 *     - activations and their gradients carry a scale for every
 *       128-element group taken along K, the contracted dimension; weights
 *       carry one per 128x128 tile (second paragraph);
 *     - every block scale is a power of two, i.e. it has the expressiveness
 *       of an E8M0 exponent (third paragraph);
 *     - Fprop, Dgrad and Wgrad of the QKV, attention-output and MLP
 *       projections all take this path, and the quantized input is kept for
 *       Wgrad (fourth paragraph).
 *   The Chinese study notes of the same paper, section 2.3 (table of the FP8
 *   boundary), state the same grouping and power-of-two scales, with FP32
 *   accumulation.
 *
 * Readings where the pages are silent (the same readings as the CPU oracle):
 *   - E4M3 is the OCP "fn" variant (bias 7, max 448, no infinities).
 *   - scale s = 2^e, e the smallest integer with amax <= 448 * 2^e, clamped to
 *     [-126, 127]; an all-zero group has s = 1.  s is the dequantisation
 *     multiplier (x ~ decode(q) * s) and is stored as fp32.
 *   - q = round-to-nearest-even(x / s) to E4M3, saturating at +-448 (under
 *     the rule above |x / s| never exceeds 448); the sign of zero is kept.
 *   - FP8BLK_SCALE_FP32, a numerics variant: the third paragraph of section
 *     3.2 sets the power-of-two scale of the run against the DeepSeek-V3
 *     recipe it otherwise follows, whose formula the pages do not print.  Its
 *     plainest reading: s = fl32(amax / 448) (IEEE division, so the group's
 *     largest magnitude lands on 448), s = 1 for an all-zero group, and
 *     q = round-to-nearest-even(fl32(x / s)) to E4M3, saturating at +-448
 *     (the rounded quotient of the amax itself can exceed 448 by an ulp).
 *   - out[i][j] = sum over 128-deep reduction blocks b of
 *       sa(i, b) * sb(j, b) * sum_{r in b} dec(A[i][r]) * dec(B[j][r]),
 *     accumulated in fp32, rounded to bf16 (RNE) or returned as fp32.
 *
 * Conventions for every entry point:
 *   - Tensors are row-major.  bf16 values are passed as their raw 16-bit
 *     patterns (uint16_t), E4M3 codes as uint8_t, scales as float.
 *   - Dimensions and leading dimensions are in elements, int64_t.
 *   - Pointers are DEVICE pointers on the current HIP device.  The caller
 *     owns every buffer; the library allocates nothing and keeps no pointer
 *     after returning.  Its only global state is two per-device records,
 *     each set once: whether the device is a gfx950 (looked up on the first
 *     call on it) and whether a GEMM kernel's dynamic-LDS limit has been
 *     raised (on the kernel's first launch there).  Concurrent first calls
 *     only repeat the same idempotent lookup or attribute call.
 *   - Every call only enqueues work on `stream` (0 = the null stream) and
 *     never synchronises; results are valid once the stream has progressed
 *     past the call.  Outputs must not alias inputs.
 *   - Return value: FP8BLK_OK (0), or a negative FP8BLK_ERR_* code.  All
 *     argument checks run on the host before any launch: on an error nothing
 *     is enqueued and no output is touched.  No C++ exception crosses the ABI.
 *   - The scale arrays do not say which rule made them, so the GEMMs that
 *     can take either are told: fp8_block_gemm and the two backward calls
 *     take a scale_mode argument.  With FP8BLK_SCALE_FP32 they run the
 *     PROMOTE algorithm (FP8BLK_ALGO_DEFAULT is resolved to it, and an
 *     explicit FP8BLK_ALGO_SCALED_MFMA is refused with FP8BLK_ERR_ARG,
 *     because the block-scaled MFMA keeps only a scale's exponent field).
 *     The named Fprop / Dgrad / Wgrad functions take FP8BLK_SCALE_POW2
 *     operands only: exact powers of two in [2^-126, 2^127].
 */
#ifndef FP8BLK_H
#define FP8BLK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Scale rule of the quantizers (the readings above): POW2, the pages' rule,
 * or FP32, s = amax / 448 unconstrained.  The GEMMs that take a scale_mode
 * are told with the same values which rule made their operands' scales. */
enum fp8blk_scale_mode { FP8BLK_SCALE_POW2 = 0, FP8BLK_SCALE_FP32 = 1 };

/* GEMM output element type.  FP32_ACCUM: fp32 output that the result is
 * added to (out = fl32(out + result)), for gradients accumulated in fp32 over
 * micro-batches; the result is the one FP8BLK_OUT_FP32 would store, bit for
 * bit, so the sum is deterministic too. */
enum fp8blk_out_dtype { FP8BLK_OUT_BF16 = 0, FP8BLK_OUT_FP32 = 1, FP8BLK_OUT_FP32_ACCUM = 2 };

/* Which contraction (for fp8_block_gemm and the workspace query;
 * FP8BLK_OP_BACKWARD, Dgrad and Wgrad together, for the workspace query and
 * the two backward functions only).  FP8BLK_OP_DGRAD_W is Dgrad reading the
 * weight codes qw [N][K] as quantized instead of the transposed copy. */
enum fp8blk_op { FP8BLK_OP_FPROP = 0, FP8BLK_OP_DGRAD = 1, FP8BLK_OP_WGRAD = 2, FP8BLK_OP_BACKWARD = 3,
                 FP8BLK_OP_DGRAD_W = 4 };

/* How the per-block scale product reaches the fp32 accumulators.
 *   PROMOTE:     one MFMA per 128-deep reduction block starting from zero,
 *                then acc = fma(P, fl32(sa * sb), acc) on the vector ALU;
 *                takes any fp32 scales;
 *   SCALED_MFMA: gfx950's block-scaled MFMA multiplies each operand row by
 *                its power-of-two scale (E8M0) inside the matrix core and
 *                accumulates in place; power-of-two scales only.
 * With power-of-two scales both compute the same sum of exactly scaled block
 * products in fp32; they differ only in rounding order.  DEFAULT picks the
 * faster one (SCALED_MFMA). */
enum fp8blk_gemm_algo { FP8BLK_ALGO_DEFAULT = 0, FP8BLK_ALGO_PROMOTE = 1, FP8BLK_ALGO_SCALED_MFMA = 2 };

/* Status codes. */
enum fp8blk_status {
    FP8BLK_OK = 0,
    FP8BLK_ERR_NULL = -1,      /* a required pointer is NULL */
    FP8BLK_ERR_DIM = -2,       /* a dimension is <= 0 or not a multiple of 128 */
    FP8BLK_ERR_ALIGN = -3,     /* a pointer or leading dimension is not 16-byte aligned */
    FP8BLK_ERR_ARG = -4,       /* bad enum, leading dimension smaller than the row, or too large */
    FP8BLK_ERR_WORKSPACE = -5, /* workspace smaller than fp8_block_gemm_workspace_size() */
    FP8BLK_ERR_HIP = -6,       /* the HIP runtime reported an error at launch */
    FP8BLK_ERR_DEVICE = -7,    /* the current device is not gfx950 */
    FP8BLK_ERR_SCRATCH = -8    /* the call needs more than FP8BLK_NOALLOC_SCRATCH_BYTES of scratch */
};

/* Size of the library's static device scratch buffer (one per GPU), used by
 * fp8_block_gemm_backward_w_noalloc in place of a caller's workspace. */
#define FP8BLK_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

/*
 * Every quantizer takes scale_mode = FP8BLK_SCALE_POW2 or FP8BLK_SCALE_FP32
 * (anything else: FP8BLK_ERR_ARG); the two differ only in the scale rule.
 *
 * Row-group quantization (section 3.2, second paragraph: groups of 128 along
 * the reduction dimension).  Used for X before Fprop and for dY before Dgrad.
 *   x    [rows][cols] bf16, row stride ld_x (>= cols, multiple of 8)
 *   q    [rows][cols] E4M3 codes, row stride ld_q (>= cols, multiple of 16)
 *   s    [rows][cols/128] fp32 scales, dense
 *   rows >= 1 (any value); cols a positive multiple of 128.
 *   x and q 16-byte aligned, s 4-byte aligned.
 */
int fp8_quantize_rowgroup(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                          uint8_t *q, int64_t ld_q, float *s, int scale_mode,
                          hipStream_t stream);

/*
 * Column-group quantization: the same rule with groups of 128 consecutive
 * ROWS (tokens) of each column, the reduction dimension of Wgrad; the output
 * is written transposed so that Wgrad reads it contiguously along tokens.
 * This is the quantized copy of the input kept for Wgrad (section 3.2,
 * fourth paragraph).  colgroup(x) equals rowgroup(x^T) bit for bit.
 *   x    [rows][cols] bf16, row stride ld_x (>= cols, multiple of 8)
 *   qT   [cols][rows] E4M3 codes, row stride ld_qT (>= rows, multiple of 16)
 *   sT   [cols][rows/128] fp32 scales, dense
 *   rows and cols positive multiples of 128.
 */
int fp8_quantize_colgroup(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                          uint8_t *qT, int64_t ld_qT, float *sT, int scale_mode,
                          hipStream_t stream);

/*
 * Row groups and column groups of the same tensor in one pass: the outputs
 * of fp8_quantize_rowgroup (q, s) and of fp8_quantize_colgroup (qT, sT),
 * bit for bit, from a single read of x.  Section 3.2 (fourth paragraph) keeps
 * the quantized input for Wgrad, so both orientations of X (and of dY) are
 * needed; one read instead of two saves a third of the quantizer traffic.
 *   x    [rows][cols] bf16, row stride ld_x (>= cols, multiple of 8)
 *   q    [rows][cols] codes, row stride ld_q (>= cols, multiple of 16); s [rows][cols/128]
 *   qT   [cols][rows] codes, row stride ld_qT (>= rows, multiple of 16); sT [cols][rows/128]
 *   rows and cols positive multiples of 128.
 */
int fp8_quantize_dual(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                      uint8_t *q, int64_t ld_q, float *s,
                      uint8_t *qT, int64_t ld_qT, float *sT, int scale_mode,
                      hipStream_t stream);

/*
 * Weight block quantization (section 3.2, second paragraph: 128x128 blocks).
 *   w    [rows][cols] bf16 (rows = out features N, cols = in features K),
 *        row stride ld_w (>= cols, multiple of 8)
 *   q    [rows][cols] E4M3 codes, dense
 *   qT   optional (NULL to skip): [cols][rows] E4M3 codes, dense -- the
 *        transposed copy that fp8_block_gemm_dgrad reads (block scales are
 *        the same); fp8_block_gemm_dgrad_w reads q itself and needs none
 *   s    [rows/128][cols/128] fp32 scales, dense
 *   rows and cols positive multiples of 128.
 */
int fp8_quantize_block(const uint16_t *w, int64_t rows, int64_t cols, int64_t ld_w,
                       uint8_t *q, uint8_t *qT, float *s, int scale_mode,
                       hipStream_t stream);

/*
 * Several weights quantized in one launch, each exactly as by
 * fp8_quantize_block (the same arguments, the same results): for instance
 * all the weights of a layer, which are known when a step starts.  Saves
 * the fixed cost of a launch per weight, which dominates for small ones.
 *   jobs    host array of n_jobs descriptors (1 <= n_jobs <= 8), read before
 *           the call returns; each must pass fp8_quantize_block's checks,
 *           and the first failing one decides the status (nothing is
 *           launched then).
 */
typedef struct fp8blk_block_job {
    const uint16_t *w;      /* [rows][cols] bf16, row stride ld_w */
    int64_t rows, cols, ld_w;
    uint8_t *q;             /* [rows][cols] codes, dense */
    uint8_t *qT;            /* NULL, or [cols][rows] codes, dense */
    float *s;               /* [rows/128][cols/128] scales */
} fp8blk_block_job;

int fp8_quantize_block_batch(const fp8blk_block_job *jobs, int n_jobs, int scale_mode,
                             hipStream_t stream);

/*
 * Fprop  Y = X W^T  (section 3.2, fourth paragraph).
 *   qx [M][K] codes + sx [M][K/128]   (from fp8_quantize_rowgroup of X)
 *   qw [N][K] codes + sw [N/128][K/128] (from fp8_quantize_block of W)
 *   y  [M][N], bf16 bits (out_dtype FP8BLK_OUT_BF16) or fp32 (FP8BLK_OUT_FP32;
 *      FP8BLK_OUT_FP32_ACCUM adds to it)
 *   M, N, K positive multiples of 128; all operands dense.
 */
int fp8_block_gemm_fprop(int64_t M, int64_t N, int64_t K,
                         const uint8_t *qx, const float *sx,
                         const uint8_t *qw, const float *sw,
                         void *y, int out_dtype, hipStream_t stream);

/*
 * Dgrad  dX = dY W  (section 3.2, fourth paragraph).
 *   qdy [M][N] codes + sdy [M][N/128]  (from fp8_quantize_rowgroup of dY)
 *   qwT [K][N] codes (the transposed copy from fp8_quantize_block of W)
 *   sw  [N/128][K/128] the same block scales as Fprop
 *   dx  [M][K], bf16 bits or fp32 (or fp32 accumulated, as for Fprop)
 */
int fp8_block_gemm_dgrad(int64_t M, int64_t N, int64_t K,
                         const uint8_t *qdy, const float *sdy,
                         const uint8_t *qwT, const float *sw,
                         void *dx, int out_dtype, hipStream_t stream);

/*
 * Dgrad from the weight codes as quantized: the same contraction and result
 * as fp8_block_gemm_dgrad, but B is qw [N][K], the row-major codes of
 * fp8_quantize_block (section 3.2, fourth paragraph: the weights are
 * quantized right before the GEMMs), so the block quantizer can skip the
 * transposed copy (qT = NULL).  The kernel stages [n][k] tiles and forms its
 * operand fragments with LDS transpose reads.
 *   qdy [M][N] codes + sdy [M][N/128]; qw [N][K] codes; sw [N/128][K/128]
 *   dx  [M][K], bf16 bits or fp32 (or fp32 accumulated)
 */
int fp8_block_gemm_dgrad_w(int64_t M, int64_t N, int64_t K,
                           const uint8_t *qdy, const float *sdy,
                           const uint8_t *qw, const float *sw,
                           void *dx, int out_dtype, hipStream_t stream);

/*
 * Wgrad  dW = dY^T X  (section 3.2, fourth paragraph); the reduction runs
 * over the M tokens, so both operands are column-group quantized.
 *   qdyT [N][M] codes + sdyT [N][M/128]  (fp8_quantize_colgroup of dY)
 *   qxT  [K][M] codes + sxT  [K][M/128]  (fp8_quantize_colgroup of X)
 *   dw   [N][K], bf16 bits or fp32 (FP8BLK_OUT_FP32_ACCUM: dw += dY^T X in
 *        fp32, the usual fp32 main-gradient accumulation)
 *   workspace: device memory of at least
 *     fp8_block_gemm_workspace_size(FP8BLK_OP_WGRAD, M, N, K) bytes, 16-byte
 *     aligned, contents on entry irrelevant: fp32 partial tiles of output
 *     tiles whose reduction is shared by several workgroups, which a second
 *     kernel sums in a fixed order, so results are deterministic.  May be
 *     NULL when that size is 0.  Two calls that run at the same time need
 *     separate workspaces.
 */
int fp8_block_gemm_wgrad(int64_t M, int64_t N, int64_t K,
                         const uint8_t *qdyT, const float *sdyT,
                         const uint8_t *qxT, const float *sxT,
                         void *dw, int out_dtype,
                         void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Dgrad and Wgrad of one linear in one call (section 3.2, fourth paragraph:
 * both backward GEMMs of the layer).  Operands and outputs are exactly those
 * of fp8_block_gemm_dgrad and fp8_block_gemm_wgrad, each output with its own
 * out_dtype (FP8BLK_OUT_FP32_ACCUM allowed for both).  The two contractions
 * have the same FLOP count and run as one launch whose workgroups share out
 * the reduction work of both evenly; results equal those of the separate
 * calls up to the order in which fp32 partial sums are added
 * (deterministic).  Shapes the fused launch does not take (the 128-block
 * count of M or N not a multiple of 4, N > 16384) run as the two separate
 * contractions.
 *   scale_mode: the rule that made all the operands' scales.
 *     FP8BLK_SCALE_POW2 takes the fused launch above; FP8BLK_SCALE_FP32
 *     (amax / 448 scales) runs Dgrad and then Wgrad with the PROMOTE
 *     algorithm, which reads the whole fp32 scales.  Anything else:
 *     FP8BLK_ERR_ARG.
 *   workspace: at least fp8_block_gemm_workspace_size(FP8BLK_OP_BACKWARD,
 *     M, N, K) bytes (enough for either scale_mode), 16-byte aligned,
 *     contents on entry irrelevant; NULL when that size is 0.
 *   dx and dw must not be the same buffer (FP8BLK_ERR_ARG).
 */
int fp8_block_gemm_backward(int64_t M, int64_t N, int64_t K,
                            const uint8_t *qdy, const float *sdy,
                            const uint8_t *qwT, const float *sw,
                            const uint8_t *qdyT, const float *sdyT,
                            const uint8_t *qxT, const float *sxT,
                            void *dx, int dx_dtype, void *dw, int dw_dtype, int scale_mode,
                            void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * fp8_block_gemm_backward with Dgrad reading the weight codes qw [N][K] as
 * quantized (as fp8_block_gemm_dgrad_w does); everything else identical,
 * including the workspace (FP8BLK_OP_BACKWARD's size).
 */
int fp8_block_gemm_backward_w(int64_t M, int64_t N, int64_t K,
                              const uint8_t *qdy, const float *sdy,
                              const uint8_t *qw, const float *sw,
                              const uint8_t *qdyT, const float *sdyT,
                              const uint8_t *qxT, const float *sxT,
                              void *dx, int dx_dtype, void *dw, int dw_dtype, int scale_mode,
                              void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * fp8_block_gemm_backward_w for callers that cannot allocate memory or hand
 * over a workspace: code being captured into a HIP graph, tight training or
 * serving loops, harnesses that forbid allocation.  The same contraction,
 * kernels and results, bit for bit, as fp8_block_gemm_backward_w with any
 * sufficient workspace; the caller still passes every input and output.
 * Where the other call would use the workspace (fp32 partial tiles of output
 * tiles whose reduction several workgroups share), this one uses a static
 * device array of FP8BLK_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library:
 * each GPU the library runs on holds its own copy until the process ends.
 * The call allocates nothing, neither through HIP nor otherwise; its first
 * call on a device looks up that device's copy once.
 *   Limit: a call whose launch needs more scratch than that returns
 *     FP8BLK_ERR_SCRATCH before launching anything.  The fused launch of
 *     power-of-two scales needs at most 32 MiB at the decoder layer's
 *     shapes (it can need up to 128 MiB at other shapes, e.g. 72 MiB at
 *     M = N = 1536, K = 2560); with amax / 448 scales (the promote
 *     pair) a call needs at most 64 MiB, so it always fits.
 *   Concurrency: every call on a GPU shares that GPU's array and leaves its
 *     contents behind (nothing in it needs to start at zero: each partial
 *     tile is written in full before it is read).  Calls whose launches
 *     overlap on one GPU -- on two streams, or from two threads -- race on
 *     it and give wrong results: order them on one stream.
 */
int fp8_block_gemm_backward_w_noalloc(int64_t M, int64_t N, int64_t K,
                                      const uint8_t *qdy, const float *sdy,
                                      const uint8_t *qw, const float *sw,
                                      const uint8_t *qdyT, const float *sdyT,
                                      const uint8_t *qxT, const float *sxT,
                                      void *dx, int dx_dtype, void *dw, int dw_dtype, int scale_mode,
                                      hipStream_t stream);

/*
 * All three contractions through one entry point, with an explicit algorithm.
 *   op = FP8BLK_OP_FPROP: (a, sa, b, sb) = (qx, sx, qw, sw),    out [M][N]
 *   op = FP8BLK_OP_DGRAD: (a, sa, b, sb) = (qdy, sdy, qwT, sw), out [M][K]
 *   op = FP8BLK_OP_WGRAD: (a, sa, b, sb) = (qdyT, sdyT, qxT, sxT), out [N][K]
 *   op = FP8BLK_OP_DGRAD_W: (a, sa, b, sb) = (qdy, sdy, qw, sw), out [M][K]
 * Operand layouts, workspace and errors are as for the named functions above
 * (which are this call with FP8BLK_ALGO_DEFAULT and FP8BLK_SCALE_POW2); a
 * bad op or algo gives FP8BLK_ERR_ARG.
 *   scale_mode: the rule that made sa and sb.  FP8BLK_SCALE_POW2: any algo.
 *     FP8BLK_SCALE_FP32 (amax / 448): FP8BLK_ALGO_DEFAULT runs PROMOTE,
 *     FP8BLK_ALGO_PROMOTE is taken as is, and FP8BLK_ALGO_SCALED_MFMA gives
 *     FP8BLK_ERR_ARG (it would keep only the scales' exponent bits).
 *     Anything else: FP8BLK_ERR_ARG.
 */
int fp8_block_gemm(int op, int64_t M, int64_t N, int64_t K,
                   const uint8_t *a, const float *sa, const uint8_t *b, const float *sb,
                   void *out, int out_dtype, int algo, int scale_mode,
                   void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes that the given contraction needs at this shape (0 if none;
 * (size_t)-1 for an invalid op or shape). */
size_t fp8_block_gemm_workspace_size(int op, int64_t M, int64_t N, int64_t K);

/* Human-readable text for a status code (static storage). */
const char *fp8_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H */
