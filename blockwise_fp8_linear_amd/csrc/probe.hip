// On-box ceiling for the GEMM kernels' matrix-core work: the same
// v_mfma_scale_f32_32x32x64_f8f6f4 instruction, 16 independent 32x32
// accumulators per wave and one wave per SIMD (the GEMM's layout), issued
// back to back on register operands -- no loads, no LDS, no epilogue.  The
// operands are pseudo-random finite E4M3 codes (the matrix core's power,
// hence its clock, depends on the data), the scales 2^0.  Used by the
// benchmark to state achieved throughput against what the chip sustains,
// besides the published peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8blk_device.h"
#include "fp8probe.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {  // an integer hash (xorshift-multiply)
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, uint32_t seed, float* out) {
  const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
  v8i a[4], b[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      // clearing bit 3 of every byte keeps the codes finite (no S.1111.111)
      a[t][r] = (int)(mix(seed ^ (gid * 64 + t * 8 + r)) & 0xF7F7F7F7u);
      b[t][r] = (int)(mix(~seed ^ (gid * 64 + t * 8 + r)) & 0xF7F7F7F7u);
    }
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  constexpr int kOne = 127;  // E8M0 scale byte of 2^0
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, kOne, 0, kOne);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  out[gid] = s;
}

// Every element a quantizer under the amax / 448 rule can see: block
// (x, y) takes the group amax with bf16 bits y (0 .. 0x7F7F, every
// non-negative finite value) and thread t the magnitude bits
// m = 256 x + t <= y, with both signs.  The quantizers' reciprocal-based
// quotient (Fp32Scale) and a plain IEEE division (Fp32ScaleDiv) must give
// the same stored scale and the same E4M3 code; each block writes how many
// of its threads found a difference.
__global__ __launch_bounds__(256) void quotient_check_kernel(uint32_t* counts) {
  const uint32_t a = blockIdx.y, m = blockIdx.x * 256 + threadIdx.x;
  bool bad = false;
  if (m <= a) {
    const fp8blk::Fp32Scale fast(a);
    const fp8blk::Fp32ScaleDiv ref(a);
    const float xp = __uint_as_float(m << 16);
    const int cf = __builtin_amdgcn_cvt_pk_fp8_f32(fast(xp), fast(-xp), 0, false);
    const int cr = __builtin_amdgcn_cvt_pk_fp8_f32(ref(xp), ref(-xp), 0, false);
    bad = ((cf ^ cr) & 0xFFFF) != 0 || __float_as_uint(fast.s) != __float_as_uint(ref.s);
  }
  const int n = __syncthreads_count(bad);
  if (threadIdx.x == 0) counts[blockIdx.y * gridDim.x + blockIdx.x] = (uint32_t)n;
}

// The power-of-two quantizers' conversion (cvt2_pow2: v_cvt_scalef32_pk_fp8_bf16
// given the stored scale 2^e) against the fp32 path it replaces (the exact
// product x * 2^-e rounded by cvt_pk_fp8_f32), for every bf16 pattern x
// (thread t of block (b, y): bits 256 b + t, in both halves of the word) and
// every scale exponent e = y - 126, -126 <= e <= 126, wherever |x| * 2^-e <=
// 448 (the codes of a finite x the rule can produce).  Each block writes
// how many of its threads found a difference.
__global__ __launch_bounds__(256) void pow2_cvt_check_kernel(uint32_t* counts) {
  const uint32_t bits = blockIdx.x * 256 + threadIdx.x;
  const int e = (int)blockIdx.y - 126;
  const float s = __builtin_ldexpf(1.0f, e), inv = __builtin_ldexpf(1.0f, -e);
  const float x = __uint_as_float(bits << 16);
  const float v = x * inv;
  bool bad = false;
  if (__builtin_isfinite(x) && __builtin_fabsf(v) <= 448.0f) {
    const uint32_t ref = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFFFFu;
    const uint32_t got = fp8blk::cvt2_pow2<false>(0u, bits | (bits << 16), s) & 0xFFFFu;
    const uint32_t got_hi = fp8blk::cvt2_pow2<true>(0u, bits | (bits << 16), s) >> 16;
    bad = got != ref || got_hi != ref;
  }
  const int n = __syncthreads_count(bad);
  if (threadIdx.x == 0) counts[blockIdx.y * gridDim.x + blockIdx.x] = (uint32_t)n;
}

// On-box HBM ceiling: streaming kernels over one buffer, each lane moving
// kStreamUnroll 16-byte pieces per step (all loads issued before the first
// store or use), non-temporal loads and stores, a grid-stride loop over
// 16-byte pieces.  copy: read src, write dst (as many bytes written as read,
// the quantizers' ratio); read: read src only, folded into one word per
// thread so that the loads are kept.
constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(256) void copy_probe_kernel(const fp8blk::u32x4* __restrict__ src,
                                                         fp8blk::u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 * kStreamUnroll + threadIdx.x; i0 < n16;
       i0 += stride * kStreamUnroll) {
    fp8blk::u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * 256;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * 256;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

__global__ __launch_bounds__(256) void read_probe_kernel(const fp8blk::u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 * kStreamUnroll + threadIdx.x; i0 < n16;
       i0 += stride * kStreamUnroll) {
    fp8blk::u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * 256;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : fp8blk::u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" int fp8probe_stream(int mode, const void* src, void* dst, size_t bytes, int workgroups,
                               hipStream_t stream) {
  if (src == nullptr || dst == nullptr || bytes == 0 || bytes % 16 != 0 || workgroups <= 0 || (mode != 0 && mode != 1))
    return -1;
  if (((uintptr_t)src & 15) != 0 || ((uintptr_t)dst & 15) != 0) return -1;
  const int64_t n16 = (int64_t)(bytes / 16);
  const auto* s = static_cast<const fp8blk::u32x4*>(src);
  if (mode == 0)
    hipLaunchKernelGGL(copy_probe_kernel, dim3((uint32_t)workgroups), dim3(256), 0, stream, s,
                       static_cast<fp8blk::u32x4*>(dst), n16);
  else
    hipLaunchKernelGGL(read_probe_kernel, dim3((uint32_t)workgroups), dim3(256), 0, stream, s, n16,
                       static_cast<uint32_t*>(dst));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int fp8probe_fp32_quotient_check(uint32_t* counts, hipStream_t stream) {
  if (counts == nullptr) return -1;
  hipLaunchKernelGGL(quotient_check_kernel, dim3(128, 0x7F80), dim3(256), 0, stream, counts);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int fp8probe_pow2_cvt_check(uint32_t* counts, hipStream_t stream) {
  if (counts == nullptr) return -1;
  hipLaunchKernelGGL(pow2_cvt_check_kernel, dim3(256, 253), dim3(256), 0, stream, counts);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int fp8probe_mfma(int workgroups, int iters, uint32_t seed, float* out, hipStream_t stream) {
  if (workgroups <= 0 || iters <= 0 || out == nullptr) return -1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((uint32_t)workgroups), dim3(256), 0, stream, iters, seed, out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" double fp8probe_mfma_flops(int workgroups, int iters) {
  // 4 waves x 16 instructions x 2*32*32*64 FLOP per iteration per workgroup
  return (double)workgroups * iters * 4.0 * 16.0 * 2.0 * 32 * 32 * 64;
}
