// C ABI of libfp8blk: argument validation and dispatch.  The contract of each
// entry point is documented in include/fp8blk.h.
#include "../../include/fp8blk.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "fp8blk_launch.h"

namespace {

constexpr int64_t kGroup = 128;
constexpr int kMaxDevices = 64;
// Once-initialised per-device answer to "is this a gfx950?": 0 unknown, 1 yes, 2 no.
std::atomic<int> g_device_ok[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool mult128(int64_t v) { return v > 0 && v % kGroup == 0; }
// a * b <= limit for a, b > 0, without forming the (possibly overflowing) product
bool prod_le(int64_t a, int64_t b, int64_t limit) { return a <= limit / b; }
// a * b < limit, likewise
bool prod_lt(int64_t a, int64_t b, int64_t limit) { return a < (limit + b - 1) / b; }
bool valid_scale_mode(int m) { return m == FP8BLK_SCALE_POW2 || m == FP8BLK_SCALE_FP32; }

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8BLK_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FP8BLK_ERR_DEVICE;
  int known = g_device_ok[dev].load(std::memory_order_acquire);
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8BLK_ERR_HIP;
    known = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_ok[dev].store(known, std::memory_order_release);
  }
  return known == 1 ? FP8BLK_OK : FP8BLK_ERR_DEVICE;
}

int finish(hipError_t e) { return e == hipSuccess ? FP8BLK_OK : FP8BLK_ERR_HIP; }

// Largest element count the 32-bit index arithmetic inside the kernels covers.
constexpr int64_t kMaxElems = int64_t(1) << 40;

}  // namespace

extern "C" {

const char* fp8_status_string(int status) {
  switch (status) {
    case FP8BLK_OK: return "ok";
    case FP8BLK_ERR_NULL: return "fp8blk: a required pointer is NULL";
    case FP8BLK_ERR_DIM: return "fp8blk: a dimension is <= 0 or not a multiple of 128";
    case FP8BLK_ERR_ALIGN: return "fp8blk: a pointer or leading dimension is not 16-byte aligned";
    case FP8BLK_ERR_ARG: return "fp8blk: bad enum value, leading dimension smaller than the row, or size too large";
    case FP8BLK_ERR_WORKSPACE: return "fp8blk: workspace smaller than fp8_block_gemm_workspace_size()";
    case FP8BLK_ERR_HIP: return "fp8blk: HIP runtime error at launch";
    case FP8BLK_ERR_DEVICE: return "fp8blk: the current device is not gfx950";
    case FP8BLK_ERR_SCRATCH:
      return "fp8blk: the call needs more scratch than the library's static buffer (FP8BLK_NOALLOC_SCRATCH_BYTES) holds";
    default: return "fp8blk: unknown status";
  }
}

int fp8_quantize_rowgroup(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                          float* s, int scale_mode, hipStream_t stream) {
  if (!valid_scale_mode(scale_mode)) return FP8BLK_ERR_ARG;
  if (!x || !q || !s) return FP8BLK_ERR_NULL;
  if (rows <= 0 || !mult128(cols)) return FP8BLK_ERR_DIM;
  if (ld_x < cols || ld_q < cols) return FP8BLK_ERR_ARG;
  if (!prod_lt(rows, cols / kGroup, int64_t(1) << 31) || !prod_le(rows, ld_x, kMaxElems) ||
      !prod_le(rows, ld_q, kMaxElems))
    return FP8BLK_ERR_ARG;
  if (!aligned16(x) || !aligned16(q) || !aligned4(s) || ld_x % 8 || ld_q % 16) return FP8BLK_ERR_ALIGN;
  if (int rc = check_device()) return rc;
  return finish(fp8blk::launch_quant_rowgroup(x, rows, cols, ld_x, q, ld_q, s, scale_mode == FP8BLK_SCALE_FP32, stream));
}

int fp8_quantize_colgroup(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qT, int64_t ld_qT,
                          float* sT, int scale_mode, hipStream_t stream) {
  if (!valid_scale_mode(scale_mode)) return FP8BLK_ERR_ARG;
  if (!x || !qT || !sT) return FP8BLK_ERR_NULL;
  if (!mult128(rows) || !mult128(cols)) return FP8BLK_ERR_DIM;
  if (ld_x < cols || ld_qT < rows) return FP8BLK_ERR_ARG;
  if (!prod_lt(rows / 128, cols / 64, int64_t(1) << 31) || !prod_le(rows, ld_x, kMaxElems) ||
      !prod_le(cols, ld_qT, kMaxElems))
    return FP8BLK_ERR_ARG;
  if (!aligned16(x) || !aligned16(qT) || !aligned4(sT) || ld_x % 8 || ld_qT % 16) return FP8BLK_ERR_ALIGN;
  if (int rc = check_device()) return rc;
  return finish(fp8blk::launch_quant_colgroup(x, rows, cols, ld_x, qT, ld_qT, sT, scale_mode == FP8BLK_SCALE_FP32, stream));
}

int fp8_quantize_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q, float* s,
                      uint8_t* qT, int64_t ld_qT, float* sT, int scale_mode, hipStream_t stream) {
  if (!valid_scale_mode(scale_mode)) return FP8BLK_ERR_ARG;
  if (!x || !q || !s || !qT || !sT) return FP8BLK_ERR_NULL;
  if (!mult128(rows) || !mult128(cols)) return FP8BLK_ERR_DIM;
  if (ld_x < cols || ld_q < cols || ld_qT < rows) return FP8BLK_ERR_ARG;
  if (!prod_lt(rows / 128, cols / 128, int64_t(1) << 31) || !prod_le(rows, ld_x, kMaxElems) ||
      !prod_le(rows, ld_q, kMaxElems) || !prod_le(cols, ld_qT, kMaxElems))
    return FP8BLK_ERR_ARG;
  if (!aligned16(x) || !aligned16(q) || !aligned16(qT) || !aligned4(s) || !aligned4(sT) || ld_x % 8 || ld_q % 16 ||
      ld_qT % 16)
    return FP8BLK_ERR_ALIGN;
  if (int rc = check_device()) return rc;
  return finish(fp8blk::launch_quant_dual(x, rows, cols, ld_x, q, ld_q, s, qT, ld_qT, sT, scale_mode == FP8BLK_SCALE_FP32,
                                              stream));
}

static int check_block(const uint16_t* w, int64_t rows, int64_t cols, int64_t ld_w, const uint8_t* q,
                       const uint8_t* qT, const float* s, int scale_mode) {
  if (!valid_scale_mode(scale_mode)) return FP8BLK_ERR_ARG;
  if (!w || !q || !s) return FP8BLK_ERR_NULL;
  if (!mult128(rows) || !mult128(cols)) return FP8BLK_ERR_DIM;
  if (ld_w < cols) return FP8BLK_ERR_ARG;
  if (!prod_lt(rows / 128, cols / 128, int64_t(1) << 31) || !prod_le(rows, ld_w, kMaxElems) ||
      !prod_le(rows, cols, kMaxElems))
    return FP8BLK_ERR_ARG;
  if (!aligned16(w) || !aligned16(q) || (qT && !aligned16(qT)) || !aligned4(s) || ld_w % 8) return FP8BLK_ERR_ALIGN;
  return FP8BLK_OK;
}

int fp8_quantize_block(const uint16_t* w, int64_t rows, int64_t cols, int64_t ld_w, uint8_t* q, uint8_t* qT,
                       float* s, int scale_mode, hipStream_t stream) {
  if (int rc = check_block(w, rows, cols, ld_w, q, qT, s, scale_mode)) return rc;
  if (int rc = check_device()) return rc;
  return finish(fp8blk::launch_quant_block(w, rows, cols, ld_w, q, qT, s, scale_mode == FP8BLK_SCALE_FP32, stream));
}

int fp8_quantize_block_batch(const fp8blk_block_job* jobs, int n_jobs, int scale_mode, hipStream_t stream) {
  if (!jobs) return FP8BLK_ERR_NULL;
  if (n_jobs < 1 || n_jobs > fp8blk::kMaxBlockJobs) return FP8BLK_ERR_ARG;
  fp8blk::BlockJob job[fp8blk::kMaxBlockJobs];
  int64_t blocks = 0;
  for (int k = 0; k < n_jobs; ++k) {
    const fp8blk_block_job& j = jobs[k];
    if (int rc = check_block(j.w, j.rows, j.cols, j.ld_w, j.q, j.qT, j.s, scale_mode)) return rc;
    blocks += (j.rows / 128) * (j.cols / 128);
    job[k] = fp8blk::BlockJob{j.w, j.rows, j.cols, j.ld_w, j.q, j.qT, j.s};
  }
  if (blocks >= (int64_t(1) << 31)) return FP8BLK_ERR_ARG;
  if (int rc = check_device()) return rc;
  return finish(fp8blk::launch_quant_block_batch(job, n_jobs, scale_mode == FP8BLK_SCALE_FP32, stream));
}

static int check_gemm_common(int64_t M, int64_t N, int64_t K, const void* a, const float* sa, const void* b,
                             const float* sb, const void* out, int out_dtype) {
  if (out_dtype != FP8BLK_OUT_BF16 && out_dtype != FP8BLK_OUT_FP32 && out_dtype != FP8BLK_OUT_FP32_ACCUM)
    return FP8BLK_ERR_ARG;
  if (!a || !sa || !b || !sb || !out) return FP8BLK_ERR_NULL;
  if (!mult128(M) || !mult128(N) || !mult128(K)) return FP8BLK_ERR_DIM;
  if (M / 128 >= (1 << 20) || N / 128 >= (1 << 20) || K / 128 >= (1 << 20) || !prod_le(M, N, kMaxElems) ||
      !prod_le(M, K, kMaxElems) || !prod_le(N, K, kMaxElems))
    return FP8BLK_ERR_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(out) || !aligned4(sa) || !aligned4(sb)) return FP8BLK_ERR_ALIGN;
  return FP8BLK_OK;
}

// The algorithm FP8BLK_ALGO_DEFAULT resolves to.
constexpr fp8blk::GemmAlgo kDefaultAlgo = fp8blk::GemmAlgo::ScaledMfma;

// The kernel-side description of one contraction (arguments already checked).
static fp8blk::GemmArgs make_args(int op, int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                                  const uint8_t* b, const float* sb, void* out, int out_dtype) {
  fp8blk::GemmArgs g{};
  g.a = a; g.sa = sa; g.b = b; g.sb = sb;
  g.out = out; g.out_f32 = out_dtype != FP8BLK_OUT_BF16; g.accumulate = out_dtype == FP8BLK_OUT_FP32_ACCUM;
  if (op == FP8BLK_OP_FPROP) {
    // Y[m][n] = sum_k X[m][k] W[n][k]; weight block (n/128, k/128)
    g.I = M; g.J = N; g.R = K;
    g.sb_j = K / kGroup; g.sb_r = 1; g.bmode = fp8blk::BScale::Block;
  } else if (op == FP8BLK_OP_DGRAD || op == FP8BLK_OP_DGRAD_W) {
    // dX[m][k] = sum_n dY[m][n] W[n][k]: B = qwT [K][N] (DGRAD) or qw [N][K]
    // read as quantized (DGRAD_W); the weight block holding (n, k) has
    // scale sw[(n/128) * (K/128) + k/128]
    g.I = M; g.J = K; g.R = N;
    g.sb_j = 1; g.sb_r = K / kGroup; g.bmode = fp8blk::BScale::Block;
    g.bt = op == FP8BLK_OP_DGRAD_W;
  } else {
    // dW[n][k] = sum_m dY[m][n] X[m][k]: A = qdyT [N][M], B = qxT [K][M]
    g.I = N; g.J = K; g.R = M;
    g.sb_j = 0; g.sb_r = 0; g.bmode = fp8blk::BScale::Row;
  }
  return g;
}

// The kernel algorithm for an (algo, scale_mode) pair, or -1 for a pair that
// cannot run: amax / 448 scales are not powers of two, and the block-scaled
// MFMA would keep only their exponent fields.
static int resolve_algo(int algo, int scale_mode, fp8blk::GemmAlgo* out) {
  if (algo != FP8BLK_ALGO_DEFAULT && algo != FP8BLK_ALGO_PROMOTE && algo != FP8BLK_ALGO_SCALED_MFMA) return -1;
  if (!valid_scale_mode(scale_mode)) return -1;
  if (scale_mode == FP8BLK_SCALE_FP32) {
    if (algo == FP8BLK_ALGO_SCALED_MFMA) return -1;
    *out = fp8blk::GemmAlgo::Promote;
    return 0;
  }
  *out = algo == FP8BLK_ALGO_PROMOTE      ? fp8blk::GemmAlgo::Promote
         : algo == FP8BLK_ALGO_SCALED_MFMA ? fp8blk::GemmAlgo::ScaledMfma
                                           : kDefaultAlgo;
  return 0;
}

int fp8_block_gemm(int op, int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa, const uint8_t* b,
                   const float* sb, void* out, int out_dtype, int algo, int scale_mode, void* workspace,
                   size_t ws_bytes, hipStream_t stream) {
  if (op != FP8BLK_OP_FPROP && op != FP8BLK_OP_DGRAD && op != FP8BLK_OP_WGRAD && op != FP8BLK_OP_DGRAD_W)
    return FP8BLK_ERR_ARG;
  fp8blk::GemmAlgo al;
  if (resolve_algo(algo, scale_mode, &al) != 0) return FP8BLK_ERR_ARG;
  if (int rc = check_gemm_common(M, N, K, a, sa, b, sb, out, out_dtype)) return rc;
  fp8blk::GemmArgs g = make_args(op, M, N, K, a, sa, b, sb, out, out_dtype);
  const size_t need = fp8blk::gemm_workspace_bytes(g.I, g.J, g.R, g.bmode);
  if (need > 0 && (workspace == nullptr || ws_bytes < need)) return FP8BLK_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return FP8BLK_ERR_ALIGN;
  if (int rc = check_device()) return rc;
  g.ws = static_cast<float*>(workspace);
  return finish(fp8blk::launch_gemm(g, al, stream));
}

// Workspace of fp8_block_gemm_backward: its own launch, or the Wgrad of the
// two-call fallback.
static size_t backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const size_t fused = fp8blk::gemm_mx_bwd_workspace_bytes(M, N, K);
  const size_t wgrad = fp8blk::gemm_workspace_bytes(N, K, M, fp8blk::BScale::Row);
  return fused > wgrad ? fused : wgrad;
}

// One backward call, checked and planned: Dgrad (gd) and Wgrad (gw), the
// algorithm, and whether they run as one fused launch.
struct BackwardCall {
  fp8blk::GemmArgs gd, gw;
  fp8blk::GemmAlgo al;
  bool fused;
};

// Checks shared by the backward entry points: dgrad_op is FP8BLK_OP_DGRAD
// (w = qwT [K][N]) or FP8BLK_OP_DGRAD_W (w = qw [N][K]).
static int backward_prepare(int dgrad_op, int64_t M, int64_t N, int64_t K, const uint8_t* qdy, const float* sdy,
                            const uint8_t* w, const float* sw, const uint8_t* qdyT, const float* sdyT,
                            const uint8_t* qxT, const float* sxT, void* dx, int dx_dtype, void* dw, int dw_dtype,
                            int scale_mode, BackwardCall* c) {
  if (!valid_scale_mode(scale_mode)) return FP8BLK_ERR_ARG;
  if (int rc = check_gemm_common(M, N, K, qdy, sdy, w, sw, dx, dx_dtype)) return rc;
  if (int rc = check_gemm_common(M, N, K, qdyT, sdyT, qxT, sxT, dw, dw_dtype)) return rc;
  if (dx == dw) return FP8BLK_ERR_ARG;
  c->gd = make_args(dgrad_op, M, N, K, qdy, sdy, w, sw, dx, dx_dtype);
  c->gw = make_args(FP8BLK_OP_WGRAD, M, N, K, qdyT, sdyT, qxT, sxT, dw, dw_dtype);
  // amax / 448 scales: the promote algorithm, which reads the whole scales
  c->al = scale_mode == FP8BLK_SCALE_FP32 ? fp8blk::GemmAlgo::Promote : kDefaultAlgo;
  c->fused = c->al == fp8blk::GemmAlgo::ScaledMfma && fp8blk::gemm_mx_bwd_eligible(c->gd, c->gw);
  return FP8BLK_OK;
}

// Workspace bytes the planned launches themselves use.
static size_t backward_path_bytes(const BackwardCall& c) {
  if (c.fused) return fp8blk::gemm_mx_bwd_workspace_bytes(c.gd.I, c.gd.R, c.gd.J);
  const size_t d = fp8blk::gemm_path_workspace_bytes(c.gd, c.al), w = fp8blk::gemm_path_workspace_bytes(c.gw, c.al);
  return d > w ? d : w;
}

static int backward_run(BackwardCall& c, void* workspace, hipStream_t stream) {
  c.gd.ws = static_cast<float*>(workspace);
  c.gw.ws = static_cast<float*>(workspace);
  if (c.fused) return finish(fp8blk::launch_gemm_mx_bwd(c.gd, c.gw, stream));
  // shapes the fused launch does not take, and amax / 448 scales: the two
  // contractions in turn (on one stream, so they may share the workspace)
  if (hipError_t e = fp8blk::launch_gemm(c.gd, c.al, stream)) return finish(e);
  return finish(fp8blk::launch_gemm(c.gw, c.al, stream));
}

static int backward(int dgrad_op, int64_t M, int64_t N, int64_t K, const uint8_t* qdy, const float* sdy,
                    const uint8_t* w, const float* sw, const uint8_t* qdyT, const float* sdyT, const uint8_t* qxT,
                    const float* sxT, void* dx, int dx_dtype, void* dw, int dw_dtype, int scale_mode,
                    void* workspace, size_t ws_bytes, hipStream_t stream) {
  BackwardCall c;
  if (int rc = backward_prepare(dgrad_op, M, N, K, qdy, sdy, w, sw, qdyT, sdyT, qxT, sxT, dx, dx_dtype, dw,
                                dw_dtype, scale_mode, &c))
    return rc;
  // the documented size covers every path, whatever the operands' alignment
  const size_t need = backward_workspace_bytes(M, N, K);
  if (need > 0 && (workspace == nullptr || ws_bytes < need)) return FP8BLK_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return FP8BLK_ERR_ALIGN;
  if (int rc = check_device()) return rc;
  return backward_run(c, workspace, stream);
}

int fp8_block_gemm_backward(int64_t M, int64_t N, int64_t K, const uint8_t* qdy, const float* sdy,
                            const uint8_t* qwT, const float* sw, const uint8_t* qdyT, const float* sdyT,
                            const uint8_t* qxT, const float* sxT, void* dx, int dx_dtype, void* dw, int dw_dtype,
                            int scale_mode, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return backward(FP8BLK_OP_DGRAD, M, N, K, qdy, sdy, qwT, sw, qdyT, sdyT, qxT, sxT, dx, dx_dtype, dw, dw_dtype,
                  scale_mode, workspace, ws_bytes, stream);
}

int fp8_block_gemm_backward_w(int64_t M, int64_t N, int64_t K, const uint8_t* qdy, const float* sdy,
                              const uint8_t* qw, const float* sw, const uint8_t* qdyT, const float* sdyT,
                              const uint8_t* qxT, const float* sxT, void* dx, int dx_dtype, void* dw, int dw_dtype,
                              int scale_mode, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return backward(FP8BLK_OP_DGRAD_W, M, N, K, qdy, sdy, qw, sw, qdyT, sdyT, qxT, sxT, dx, dx_dtype, dw, dw_dtype,
                  scale_mode, workspace, ws_bytes, stream);
}

int fp8_block_gemm_backward_w_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t* qdy, const float* sdy,
                                      const uint8_t* qw, const float* sw, const uint8_t* qdyT, const float* sdyT,
                                      const uint8_t* qxT, const float* sxT, void* dx, int dx_dtype, void* dw,
                                      int dw_dtype, int scale_mode, hipStream_t stream) {
  BackwardCall c;
  if (int rc = backward_prepare(FP8BLK_OP_DGRAD_W, M, N, K, qdy, sdy, qw, sw, qdyT, sdyT, qxT, sxT, dx, dx_dtype, dw,
                                dw_dtype, scale_mode, &c))
    return rc;
  if (backward_path_bytes(c) > FP8BLK_NOALLOC_SCRATCH_BYTES) return FP8BLK_ERR_SCRATCH;
  if (int rc = check_device()) return rc;
  void* scratch = nullptr;
  size_t bytes = 0;
  if (fp8blk::static_scratch(&scratch, &bytes) != hipSuccess) return FP8BLK_ERR_HIP;
  return backward_run(c, scratch, stream);
}

int fp8_block_gemm_fprop(int64_t M, int64_t N, int64_t K, const uint8_t* qx, const float* sx, const uint8_t* qw,
                         const float* sw, void* y, int out_dtype, hipStream_t stream) {
  return fp8_block_gemm(FP8BLK_OP_FPROP, M, N, K, qx, sx, qw, sw, y, out_dtype, FP8BLK_ALGO_DEFAULT,
                        FP8BLK_SCALE_POW2, nullptr, 0, stream);
}

int fp8_block_gemm_dgrad(int64_t M, int64_t N, int64_t K, const uint8_t* qdy, const float* sdy, const uint8_t* qwT,
                         const float* sw, void* dx, int out_dtype, hipStream_t stream) {
  return fp8_block_gemm(FP8BLK_OP_DGRAD, M, N, K, qdy, sdy, qwT, sw, dx, out_dtype, FP8BLK_ALGO_DEFAULT,
                        FP8BLK_SCALE_POW2, nullptr, 0, stream);
}

int fp8_block_gemm_dgrad_w(int64_t M, int64_t N, int64_t K, const uint8_t* qdy, const float* sdy, const uint8_t* qw,
                           const float* sw, void* dx, int out_dtype, hipStream_t stream) {
  return fp8_block_gemm(FP8BLK_OP_DGRAD_W, M, N, K, qdy, sdy, qw, sw, dx, out_dtype, FP8BLK_ALGO_DEFAULT,
                        FP8BLK_SCALE_POW2, nullptr, 0, stream);
}

int fp8_block_gemm_wgrad(int64_t M, int64_t N, int64_t K, const uint8_t* qdyT, const float* sdyT,
                         const uint8_t* qxT, const float* sxT, void* dw, int out_dtype, void* workspace,
                         size_t ws_bytes, hipStream_t stream) {
  return fp8_block_gemm(FP8BLK_OP_WGRAD, M, N, K, qdyT, sdyT, qxT, sxT, dw, out_dtype, FP8BLK_ALGO_DEFAULT,
                        FP8BLK_SCALE_POW2, workspace, ws_bytes, stream);
}

size_t fp8_block_gemm_workspace_size(int op, int64_t M, int64_t N, int64_t K) {
  if (!mult128(M) || !mult128(N) || !mult128(K)) return (size_t)-1;
  if (M / 128 >= (1 << 20) || N / 128 >= (1 << 20) || K / 128 >= (1 << 20)) return (size_t)-1;
  switch (op) {
    case FP8BLK_OP_FPROP: return fp8blk::gemm_workspace_bytes(M, N, K, fp8blk::BScale::Block);
    case FP8BLK_OP_DGRAD:
    case FP8BLK_OP_DGRAD_W: return fp8blk::gemm_workspace_bytes(M, K, N, fp8blk::BScale::Block);
    case FP8BLK_OP_WGRAD: return fp8blk::gemm_workspace_bytes(N, K, M, fp8blk::BScale::Row);
    case FP8BLK_OP_BACKWARD: return backward_workspace_bytes(M, N, K);
    default: return (size_t)-1;
  }
}

}  // extern "C"
