// Internal launch entry points of libfp8blk (host side).  Arguments are
// validated by the C ABI layer (api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace fp8blk {

// fp32_scale: the scale rule of FP8BLK_SCALE_FP32 (amax / 448) instead of the
// power-of-two one.
hipError_t launch_quant_rowgroup(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                 int64_t ld_q, float* s, bool fp32_scale, hipStream_t stream);
hipError_t launch_quant_colgroup(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qT,
                                 int64_t ld_qT, float* sT, bool fp32_scale, hipStream_t stream);
hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                             float* s, uint8_t* qT, int64_t ld_qT, float* sT, bool fp32_scale, hipStream_t stream);
// One weight of a batched block quantization.
struct BlockJob {
  const uint16_t* w;
  int64_t rows, cols, ld_w;
  uint8_t* q;
  uint8_t* qT;  // may be null
  float* s;
};
constexpr int kMaxBlockJobs = 8;
hipError_t launch_quant_block_batch(const BlockJob* job, int n, bool fp32_scale, hipStream_t stream);
hipError_t launch_quant_block(const uint16_t* w, int64_t rows, int64_t cols, int64_t ld_w, uint8_t* q, uint8_t* qT,
                              float* s, bool fp32_scale, hipStream_t stream);

// How the B operand's scales are indexed.  A's scales are always per row:
// sa[i * (R/128) + rb].  B_BLOCK: sb[(j/128) * sb_j + rb * sb_r] (a 128x128
// weight block); B_ROW: sb[j * (R/128) + rb].
enum class BScale { Block, Row };

struct GemmArgs {
  int64_t I, J, R;          // out is I x J, reduction length R
  const uint8_t* a;         // [I][R]
  const float* sa;          // [I][R/128]
  const uint8_t* b;         // [J][R]
  const float* sb;
  int64_t sb_j, sb_r;       // strides for BScale::Block
  BScale bmode;
  void* out;                // [I][J]
  bool out_f32;
  bool accumulate;          // fp32 output only: out += result
  float* ws;                // stream-K workspace (may be null when none is needed)
  bool bt;                  // B stored [R][J] instead of [J][R] (Dgrad from the weight codes
                            // as quantized); weight-block scales only
};

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per device (bit d of *done set after device d succeeded; concurrent first
// calls only repeat the same idempotent call).
hipError_t ensure_lds_limit(const void* kernel, int bytes, std::atomic<uint64_t>* done);

// Workspace bytes that a contraction needs whichever kernel takes it.
size_t gemm_workspace_bytes(int64_t I, int64_t J, int64_t R, BScale bmode);

// Promote: MFMA from zero per 128-deep block, scale product applied on the
// VALU into fp32 accumulators.  ScaledMfma: the gfx950 block-scaled MFMA
// applies the power-of-two scales in the matrix core and accumulates in place.
enum class GemmAlgo { Promote, ScaledMfma };

hipError_t launch_gemm(const GemmArgs& g, GemmAlgo algo, hipStream_t stream);

// The 256x256 block-scaled-MFMA kernel (gemm_mx.hip), the shapes it takes
// and the workspace its stream-K form (B_ROW, i.e. Wgrad) needs.
bool gemm_mx_eligible(const GemmArgs& g);
size_t gemm_mx_workspace_bytes(int64_t I, int64_t J, int64_t R, BScale bmode);
hipError_t launch_gemm_mx(const GemmArgs& g, hipStream_t stream);

// Workspace bytes that launch_gemm(g, algo) itself uses (the stream-K
// partial tiles of the general kernel or of the 256x256 kernel).
size_t gemm_path_workspace_bytes(const GemmArgs& g, GemmAlgo algo);

// The library's static device scratch on the current device (scratch.hip):
// its device address and size.
hipError_t static_scratch(void** ptr, size_t* bytes);

// Dgrad (gd: I = M, J = K, R = N, weight-block scales) and Wgrad (gw: I = N,
// J = K, R = M, row scales) of one linear in one launch; the workspace is
// gw.ws.
bool gemm_mx_bwd_eligible(const GemmArgs& gd, const GemmArgs& gw);
size_t gemm_mx_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_mx_bwd(const GemmArgs& gd, const GemmArgs& gw, hipStream_t stream);

}  // namespace fp8blk
