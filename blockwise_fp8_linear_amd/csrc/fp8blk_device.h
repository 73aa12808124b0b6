// Device-side helpers shared by the gfx950 kernels of libfp8blk.
//
// Conventions follow include/fp8blk.h: bf16 values arrive as raw 16-bit
// patterns, E4M3 codes are OCP "fn" bytes, scales are fp32 multipliers --
// powers of two by default (so their exponent field is an E8M0 byte), or
// amax / 448 under FP8BLK_SCALE_FP32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// DPP controls (GFX9 encoding): rotate right within a 16-lane row, quad
// permutations, and the mirror within each 8-lane half row.
constexpr int kDppRowRor1 = 0x121;
constexpr int kDppRowRor2 = 0x122;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Largest of the two 16-bit halves, per half, of two packed words.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  ushort2_t x = __builtin_bit_cast(ushort2_t, a);
  ushort2_t y = __builtin_bit_cast(ushort2_t, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// |x| of two packed bf16 values is their bit pattern without the sign bit,
// and for non-NaN values the unsigned order of those patterns is the order
// of the magnitudes, so an integer max is an exact amax.
__device__ __forceinline__ uint32_t abs2(uint32_t w) { return w & 0x7FFF7FFFu; }

// Max over the 16 lanes of a DPP row; every lane of the row gets the result.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, dpp<kDppRowRor8>(v));
  v = max(v, dpp<kDppRowRor4>(v));
  v = max(v, dpp<kDppRowRor2>(v));
  v = max(v, dpp<kDppRowRor1>(v));
  return v;
}

// Per-half max of two packed 16-bit values over each aligned group of 8
// lanes; every lane of the group gets it.  (A 32-bit max would order by the
// high half and lose the low one.)
__device__ __forceinline__ uint32_t lane8_max_pk(uint32_t v) {
  v = pk_max_u16(v, dpp<kDppQuadSwap1>(v));
  v = pk_max_u16(v, dpp<kDppQuadSwap2>(v));
  v = pk_max_u16(v, dpp<kDppHalfMirror>(v));
  return v;
}

// Max over all 64 lanes of a wave (result in every lane).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = row16_max(v);
  v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
  return v;
}

// Scale exponent from the bf16 pattern of a non-negative amax.
// amax = (1 + m/128) * 2^(E-127) and 448 = 1.75 * 2^8, so the smallest e with
// amax <= 448 * 2^e is E - 135, plus one when m > 96.  A zero amax gives 0
// (scale 1); bf16 subnormals and everything below 448 * 2^-126 clamp to -126.
// For finite bf16 input the result lies in [-126, 120].
__device__ __forceinline__ int scale_exponent(uint32_t amax_bits) {
  int E = (int)(amax_bits >> 7);
  int m = (int)(amax_bits & 0x7F);
  int e = E - 135 + (m > 96 ? 1 : 0);
  e = e < -126 ? -126 : e;
  return amax_bits == 0 ? 0 : e;
}

// 2^e for e in [-126, 127] and 2^-e for e in [-126, 126], built from bits.
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// bf16 pattern (low or high half of a word) to fp32, exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// The two scale rules, each built from the bf16 pattern of a group's
// non-negative amax: `s` is the scale stored, and sc(x) the value that the
// element x is rounded from (the converter rounds to nearest even).
//  * Pow2Scale (the pages' run: "Puro-2B ... part 3/7", section 3.2, third
//    paragraph): s = 2^e by scale_exponent; x * 2^-e is exact and, by the
//    rule, at most 448 in magnitude, so the conversion is the only rounding.
//  * Fp32Scale (the DeepSeek-V3 representation that the same paragraph
//    contrasts with the power-of-two one): s = fl32(amax / 448), 1 for an
//    all-zero group, and the value fl32(x / s), clamped to +-448 (the cast
//    saturates; the rounded quotient of the amax itself may exceed 448 by
//    an ulp).  The scale is an IEEE-correctly rounded division.  The
//    quotient is not divided per element: y = x * r with r = fl32(1 / s),
//    then one Newton-Markstein correction y + (x - s y) r, whose residual
//    the fused multiply-add forms exactly.  Tiny scales are first brought
//    up by 2^64 together with x (both products exact, the quotient
//    unchanged), so that 1 / s cannot overflow and the residual cannot
//    underflow.  The sign is copied from x, which keeps the sign of zero.
//    Fp32ScaleDiv is the same rule with a plain division per element; the
//    measurement probe checks that the two give the same E4M3 code for
//    every bf16 amax and every bf16 x with |x| <= amax, i.e. for every
//    element a quantizer can see.
struct Pow2Scale {
  // the conversion can take the scale itself (cvt2_pow2 below)
  static constexpr bool kScaledCvt = true;
  float s, inv;
  __device__ __forceinline__ explicit Pow2Scale(uint32_t amax_bits) {
    const int e = scale_exponent(amax_bits);
    s = pow2f(e);
    inv = pow2f(-e);
  }
  __device__ __forceinline__ float operator()(float x) const { return x * inv; }
};

struct Fp32Scale {
  static constexpr bool kScaledCvt = false;
  float s;      // the stored scale
  float f;      // 2^64 if s < 2^-64, else 1
  float sf, r;  // s * f (exact) and fl32(1 / (s * f))
  __device__ __forceinline__ explicit Fp32Scale(uint32_t amax_bits) {
    s = amax_bits == 0 ? 1.0f : __uint_as_float(amax_bits << 16) / 448.0f;
    f = s < 0x1p-64f ? 0x1p64f : 1.0f;
    sf = s * f;
    r = 1.0f / sf;
  }
  __device__ __forceinline__ float operator()(float x) const {
    const float xf = x * f;
    const float y = xf * r;
    const float e = __builtin_fmaf(-sf, y, xf);
    const float v = __builtin_copysignf(__builtin_fmaf(e, r, y), x);
    return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
  }
};

struct Fp32ScaleDiv {
  static constexpr bool kScaledCvt = false;
  float s;
  __device__ __forceinline__ explicit Fp32ScaleDiv(uint32_t amax_bits) {
    s = amax_bits == 0 ? 1.0f : __uint_as_float(amax_bits << 16) / 448.0f;
  }
  __device__ __forceinline__ float operator()(float x) const {
    const float v = x / s;
    return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
  }
};

// Two bf16 (the halves of w, low half first) divided by the power-of-two
// scale s and rounded to E4M3 (RNE) in one instruction, CDNA4's
// v_cvt_scalef32_pk_fp8_bf16: the two codes go to the low (HI = false) or
// high half of the result, the other half is old's.  The instruction divides
// by 2^(exponent field of s).  Given a scale 2^e, -126 <= e <= 126 (every
// scale the power-of-two rule produces), it returns for every bf16 x with
// |x / s| <= 448 the code of the exact quotient x * 2^-e rounded to nearest
// even: fp8probe_pow2_cvt_check compares it with cvt_pk_fp8_f32 of the
// exact product over all 65536 bf16 patterns at every such e and finds no
// difference.  It replaces the unpacking to fp32, the multiply and the
// conversion of two values.
typedef short v2i16_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t cvt2_pow2(uint32_t old, uint32_t w, float s) {
  const v2i16_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(v2i16_t, old),
                                                              __builtin_bit_cast(v2bf16_t, w), s, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Four bf16 (two words) scaled by sc and rounded to E4M3 (RNE) into one
// word, byte i holding element i.
template <class S>
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, const S& sc) {
  if constexpr (S::kScaledCvt) {
    return cvt2_pow2<true>(cvt2_pow2<false>(0u, w0, sc.s), w1, sc.s);
  } else {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(sc(bf16_lo(w0)), sc(bf16_hi(w0)), 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(sc(bf16_lo(w1)), sc(bf16_hi(w1)), r, true);
    return (uint32_t)r;
  }
}

// Same for four values given as lo/hi halves of four different words
// (used where a word holds two columns).
template <class S>
__device__ __forceinline__ uint32_t quant4_sel(float a, float b, float c, float d, const S& sc) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(sc(a), sc(b), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(sc(c), sc(d), r, true);
  return (uint32_t)r;
}

// One column of four rows: wi holds row i's value in its half H (0: low
// 16 bits), all with the scale sc; byte i of the result is row i's code.
// With a power-of-two scale each pair of rows is gathered into one word
// (v_perm_b32) and converted by the scaled instruction.
template <int H, class S>
__device__ __forceinline__ uint32_t quant4_col(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, const S& sc) {
  if constexpr (S::kScaledCvt) {
    constexpr uint32_t sel = H ? 0x07060302u : 0x05040100u;  // half H of the low word, then of the high word
    // the gathered word is dead after the conversion, so it also serves as
    // the half that the second conversion overwrites (no register to clear)
    const uint32_t p01 = __builtin_amdgcn_perm(w1, w0, sel);
    const uint32_t r = cvt2_pow2<false>(p01, p01, sc.s);
    return cvt2_pow2<true>(r, __builtin_amdgcn_perm(w3, w2, sel), sc.s);
  } else {
    const auto f = [](uint32_t w) { return H ? bf16_hi(w) : bf16_lo(w); };
    return quant4_sel(f(w0), f(w1), f(w2), f(w3), sc);
  }
}

// 4x4 byte transpose: in[r] holds bytes (r,0..3); out[c] gets bytes (0..3,c).
__device__ __forceinline__ void transpose4x4(const uint32_t in[4], uint32_t out[4]) {
  uint32_t a = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);  // r0c0 r1c0 r0c1 r1c1
  uint32_t b = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);  // r0c2 r1c2 r0c3 r1c3
  uint32_t c = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);  // r2c0 r3c0 r2c1 r3c1
  uint32_t d = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);  // r2c2 r3c2 r2c3 r3c3
  out[0] = __builtin_amdgcn_perm(c, a, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(c, a, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(d, b, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(d, b, 0x07060302u);
}

// ds_read_b64_tr_b8 (gfx950), as probed on the GPU: within each group of 16
// lanes, lane i receives, as byte b, byte i % 8 of the 8 bytes addressed by
// lane 2 b + i / 8 of the group.  With lanes 2b and 2b+1 addressing row b of
// a [reduction][column] tile in LDS at columns c..c+7 and c+8..c+15, lane i
// gets column c + i and the 8 consecutive reduction values of rows 0..7 --
// an MFMA operand fragment of a tile stored along the reduction's rows.
typedef int v2i_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2i_t lds_read_tr8(const uint8_t* p) {
  typedef __attribute__((address_space(3))) v2i_t lds_v2i;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)((const __attribute__((address_space(3))) uint8_t*)p));
}

// Two fp32 values rounded to bf16 (nearest even), packed: lo in bits 15:0.
// One v_cvt_pk_bf16_f32 on gfx950.
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const v2bf_t b = __builtin_convertvector((v2f_t{lo, hi}), v2bf_t);
  return __builtin_bit_cast(uint32_t, b);
}

// XCD-aware remap of a linear workgroup id.  Consecutive ids are dealt to the
// 8 XCDs in turn; this makes each XCD own a contiguous range of logical ids
// (when the count divides evenly) so neighbouring tiles share an L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblocks) {
  constexpr uint32_t kXcds = 8;
  if (nblocks % kXcds != 0) return bid;
  return (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
}

// 16-byte direct global->LDS load: lane p's 16 bytes from base + voff land at
// LDS offset lds_addr + 16 p (lds_addr wave-uniform, in M0).  Written as
// inline assembly on purpose: the compiler would otherwise treat every
// later LDS read as depending on every such load and drain them all
// (vmcnt(0)) before it, which defeats loading ahead.  The GEMM kernels wait
// for these loads themselves with explicit vmcnt counts.  The block has no
// register outputs; it sets M0 itself, and those kernels have no other M0
// users.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds_addr) {
  // the base is wave-uniform but may have been computed in vector registers
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  // (readfirstlane returns int: go through uint32_t so the low half is not
  // sign-extended into the high half)
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// 4-byte variant: lane p's dword lands at lds_addr + 4 p.
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t voff, uint32_t lds_addr) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sb),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// The LDS byte address of a pointer into the workgroup's shared memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt low 4 bits and
// bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS only.  (__syncthreads() also waits for
// every outstanding global access, which would drain loads issued ahead of
// time; those are waited for where their data is used.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace fp8blk
