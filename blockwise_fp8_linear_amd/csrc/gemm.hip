// Block-scaled FP8 GEMM for gfx950:  out[i][j] = sum over 128-deep reduction
// blocks b of sa(i,b) * sb(j,b) * sum_{r in b} A[i][r] * B[j][r]
// with E4M3 operands, fp32 accumulation and bf16 (RNE) or fp32 output.
//
// This one "TN" kernel serves the three contractions of the FP8 linear layer
// ("Puro-2B ... part 3/7", section 3.2, fourth paragraph: Fprop, Dgrad and
// Wgrad all on the FP8 path): both operands are stored contiguous along the
// reduction dimension, so
//   Fprop  Y  = X W^T : A = qx   [M][K], B = qw  [N][K], B scales per block
//   Dgrad  dX = dY W  : A = qdy  [M][N], B = qwT [K][N], B scales per block
//                       (or B = qw [N][K] as quantized: the BT configurations)
//   Wgrad  dW = dY^T X: A = qdyT [N][M], B = qxT [K][M], B scales per row
// (one scale per 128 along the reduction dimension for activations and
// gradients, per 128x128 block for weights: section 3.2, second paragraph).
//
// Structure (per workgroup): a BM x BN output tile, the reduction walked in
// 128-deep blocks.  Each block's A and B tiles (BM x 128 and BN x 128 bytes)
// go to LDS by direct global->LDS loads, double buffered (the next block
// loads while this one is computed), with the 16-byte chunks of a row
// XOR-swizzled by (row & 7) so that the MFMA fragment reads are free of bank
// conflicts.  One v_mfma_*_16x16x128_f8f6f4 consumes exactly one 128-deep
// block for a 16x16 sub-tile, so the per-block scale product is applied
// between blocks:
//   PROMOTE = true : P = MFMA(A_b, B_b) from zero, then
//                    acc = fma(P, fl32(sa*sb), acc) on the VALU, in fp32 --
//                    any fp32 scales, so it also serves the amax / 448 rule;
//                    each sub-tile's promotion runs three MFMAs behind its
//                    MFMA, so the matrix core and the VALU overlap;
//   PROMOTE = false: the gfx950 block-scaled MFMA, which multiplies each
//                    operand row by its power-of-two scale (an E8M0 byte:
//                    the fp32 scale's exponent field) inside the matrix core
//                    and accumulates in place.
// The MFMA operands are swapped (B tile as the instruction's A operand) so
// that each lane ends up holding 4 consecutive output columns of one row,
// which makes the scale a single value per lane (per row) for the weight
// block case and the epilogue a row-contiguous 8- or 16-byte store.
// Scales of a chunk of up to kChunk reduction blocks are staged in LDS, as
// fp32 values (PROMOTE) or E8M0 bytes (the scaled MFMA).
#include <type_traits>

#include "fp8blk_device.h"
#include "fp8blk_launch.h"

namespace fp8blk {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kChunk = 32;  // reduction blocks whose scales sit in LDS at once

// BT_: B stored [R][J] (Dgrad from the weight codes as quantized): the B
// tile is staged as 128 reduction rows of BN bytes and its fragments come
// from LDS transpose reads.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, bool PROMOTE_, bool BROW_, bool BT_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr bool BT = BT_;
  static_assert(!BT_ || (!BROW_ && BN_ == 128), "transposed B: Dgrad's weight-block layout, 128-byte rows");
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr bool PROMOTE = PROMOTE_, BROW = BROW_;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  // one staged scale: fp32 for PROMOTE, its E8M0 byte for the scaled MFMA
  using SType = typename std::conditional<PROMOTE_, float, uint8_t>::type;
  static constexpr int SA_BYTES = kChunk * BM * (int)sizeof(SType);
  static constexpr int SB_BYTES = (BROW ? kChunk * BN : kChunk * (BN / 128 > 0 ? BN / 128 : 1)) * (int)sizeof(SType);
  static constexpr int LDS = 2 * STAGE + SA_BYTES + ((SB_BYTES + 15) / 16) * 16;
  static_assert(A_BYTES % (1024 * (THREADS / 64)) == 0 && B_BYTES % (1024 * (THREADS / 64)) == 0,
                "whole KiB of direct loads per wave");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must sit inside one 128-block");
  static_assert(TM % 4 == 0 || TM < 4, "scale bytes are read in words");
};

__device__ __forceinline__ uint32_t e8_of(float s) { return (__float_as_uint(s) >> 23) & 0xFFu; }

// A scale as staged in LDS by configuration C.
template <class C>
__device__ __forceinline__ typename C::SType staged_scale(float s) {
  if constexpr (C::PROMOTE) return s;
  else return (uint8_t)e8_of(s);
}

// Read a 32-byte MFMA fragment of a transposed-B tile ([128 reduction
// rows][128 B of columns], 16-byte chunks swizzled by row & 7): the lane's
// column is 16 * col16 + lane % 16 and its reduction values are
// 32 (lane / 16) .. +31, the order of read_frag's; four transpose reads of 8
// rows each (see lds_read_tr8).  Row n = 32 q + 8 r + s / 2 of lane group
// q, position s, so n & 7 = s / 2.
__device__ __forceinline__ v8i read_frag_bt(const uint8_t* tile, uint32_t col16, uint32_t lane) {
  const uint32_t q = lane >> 4, s = lane & 15;
  const uint8_t* p = tile + (32 * q + (s >> 1)) * 128 + ((col16 ^ (s >> 1)) << 4) + 8 * (s & 1);
  v8i f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const v2i_t v = lds_read_tr8(p + r * 8 * 128);
    f[2 * r] = v[0];
    f[2 * r + 1] = v[1];
  }
  return f;
}

// Read a 32-byte MFMA fragment: row `row` of a swizzled [rows][128 B] tile,
// logical 16-byte chunks 2g and 2g+1.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, uint32_t row, uint32_t g) {
  const uint32_t sw = row & 7;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + row * 128 + (((2 * g) ^ sw) << 4));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + row * 128 + (((2 * g + 1) ^ sw) << 4));
  v8i f;
  f[0] = (int)lo[0]; f[1] = (int)lo[1]; f[2] = (int)lo[2]; f[3] = (int)lo[3];
  f[4] = (int)hi[0]; f[5] = (int)hi[1]; f[6] = (int)hi[2]; f[7] = (int)hi[3];
  return f;
}

// p = the product of one 128-deep block (v_mfma_f32_16x16x128_f8f6f4 from
// zero; srcA b, srcB a), into vector registers.  Inline assembly so that the
// MFMA is issued exactly here, in the promotion pipeline's order; prev, the
// product of an earlier sub-tile (untouched), passes through the statement
// so that its promotion cannot be scheduled ahead of this MFMA.  The
// compiler does not see an MFMA here, so the hazard it would handle is
// covered by the order: every product is first read three MFMAs and two
// promotions after its MFMA (more than the 12 wait states an MFMA result
// needs before a vector-ALU read; the operands come from LDS reads, which
// the compiler waits for).
__device__ __forceinline__ void mfma16_zero(v4f& p, const v8i& b, const v8i& a) {
  asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(p) : "v"(b), "v"(a));
}
__device__ __forceinline__ void mfma16_zero(v4f& p, const v8i& b, const v8i& a, v4f& prev) {
  asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %2, %3, 0" : "=&v"(p), "+v"(prev) : "v"(b), "v"(a));
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_kernel(GemmArgs g, int64_t tiles_m, int64_t tiles_n,
                                                          int64_t kb_per_split) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* const tiles = lds;
  typedef typename C::SType ST;
  ST* const sa_lds = reinterpret_cast<ST*>(lds + 2 * C::STAGE);
  ST* const sb_lds = reinterpret_cast<ST*>(lds + 2 * C::STAGE + C::SA_BYTES);

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const uint32_t l16 = lane & 15, g4 = lane >> 4;

  // ---- which tile / split this workgroup owns
  const int64_t ntiles = tiles_m * tiles_n;
  const uint32_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t split = L / ntiles;
  const int64_t tile = L - split * ntiles;
  constexpr int64_t GM = 8;
  const int64_t group = tile / (GM * tiles_n);
  const int64_t first_m = group * GM;
  const int64_t gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int64_t in_group = tile - group * GM * tiles_n;
  const int64_t tm = first_m + in_group % gsize;
  const int64_t tn = in_group / gsize;
  const int64_t i0 = tm * C::BM, j0 = tn * C::BN;

  const int64_t nkb = g.R / 128;
  const int64_t kb_begin = split * kb_per_split;
  const int64_t kb_end = (kb_begin + kb_per_split) < nkb ? (kb_begin + kb_per_split) : nkb;
  const int64_t R = g.R;

  // ---- direct global->LDS loads of one reduction block's tiles into stage
  // buf.  Wave instruction u fills 8 rows x 128 B: lane p writes LDS bytes
  // 16 p of that KiB, row p/8, physical chunk p%8, which holds logical chunk
  // (p%8) ^ (row & 7).  Rows past an edge read the last row (BT: chunks past
  // the column edge read the last valid one); their results are never stored.
  // Each instruction has its own wave-uniform base at its first row, so the
  // per-lane 32-bit offsets stay below 8 rows (the reduction length is
  // unrestricted here).
  constexpr int A_DMA = C::A_BYTES / 1024 / (C::THREADS / 64), B_DMA = C::B_BYTES / 1024 / (C::THREADS / 64);
  const uint32_t lds0 = lds_offset(lds);
  const uint8_t* baseA[A_DMA];
  const uint8_t* baseB[B_DMA];
  uint32_t offA[A_DMA], offB[B_DMA];
#pragma unroll
  for (int u = 0; u < A_DMA; ++u) {
    const uint32_t r8 = (wave * A_DMA + u) * 8, row = r8 + (lane >> 3);
    const int64_t g0 = (i0 + r8) < g.I ? (i0 + r8) : g.I - 1;
    const int64_t gr = (i0 + row) < g.I ? (i0 + row) : g.I - 1;
    baseA[u] = g.a + g0 * R;
    offA[u] = (uint32_t)((gr - g0) * R) + (((lane & 7) ^ (row & 7)) << 4);
  }
#pragma unroll
  for (int u = 0; u < B_DMA; ++u) {
    const uint32_t r8 = (wave * B_DMA + u) * 8, row = r8 + (lane >> 3);
    if constexpr (C::BT) {
      // reduction row kb * 128 + row, columns j0 + 16 * logical chunk ..
      int64_t col = 16 * (int64_t)((lane & 7) ^ (row & 7));
      col = j0 + col < g.J - 16 ? col : g.J - 16 - j0;
      baseB[u] = g.b + (int64_t)r8 * g.J + j0;
      offB[u] = (uint32_t)((lane >> 3) * g.J + col);
    } else {
      const int64_t g0 = (j0 + r8) < g.J ? (j0 + r8) : g.J - 1;
      const int64_t gr = (j0 + row) < g.J ? (j0 + row) : g.J - 1;
      baseB[u] = g.b + g0 * R;
      offB[u] = (uint32_t)((gr - g0) * R) + (((lane & 7) ^ (row & 7)) << 4);
    }
  }
  auto dma_block = [&](int64_t kb, int buf) {
    const uint32_t st = lds0 + (uint32_t)buf * C::STAGE;
#pragma unroll
    for (int u = 0; u < A_DMA; ++u) dma16(baseA[u] + kb * 128, offA[u], st + (wave * A_DMA + u) * 1024);
#pragma unroll
    for (int u = 0; u < B_DMA; ++u)
      dma16(C::BT ? baseB[u] + kb * 128 * g.J : baseB[u] + kb * 128, offB[u],
            st + C::A_BYTES + (wave * B_DMA + u) * 1024);
  };
  // ---- scales of reduction blocks [kb0, kb0 + n) -> LDS (fp32 or E8M0).
  // sa_lds[kbl][i % 16][i / 16]; row-mode B: promote keeps [kbl][j], the
  // scaled MFMA wants [kbl][j % 16][j / 16]; block-mode B: [kbl][j / 128].
  auto load_scales = [&](int64_t kb0, int64_t n) {
    const int64_t nkb_all = nkb;
    for (uint32_t idx = tid; idx < (uint32_t)(C::BM * kChunk); idx += C::THREADS) {
      const uint32_t i = idx % C::BM, kbl = idx / C::BM;
      if (kbl < n) {
        int64_t row = i0 + i;
        row = row < g.I ? row : g.I - 1;
        sa_lds[kbl * C::BM + (i & 15) * (C::BM / 16) + (i >> 4)] = staged_scale<C>(g.sa[row * nkb_all + kb0 + kbl]);
      }
    }
    if constexpr (C::BROW) {
      for (uint32_t idx = tid; idx < (uint32_t)(C::BN * kChunk); idx += C::THREADS) {
        const uint32_t j = idx % C::BN, kbl = idx / C::BN;
        if (kbl < n) {
          int64_t row = j0 + j;
          row = row < g.J ? row : g.J - 1;
          const uint32_t pos = C::PROMOTE ? j : (j & 15) * (C::BN / 16) + (j >> 4);
          sb_lds[kbl * C::BN + pos] = staged_scale<C>(g.sb[row * nkb_all + kb0 + kbl]);
        }
      }
    } else {
      constexpr int NB = C::BN / 128;
      for (uint32_t idx = tid; idx < (uint32_t)(NB * kChunk); idx += C::THREADS) {
        const uint32_t jb = idx % NB, kbl = idx / NB;
        if (kbl < n) {
          int64_t jblk = (j0 >> 7) + jb;
          jblk = jblk < (g.J >> 7) ? jblk : (g.J >> 7) - 1;
          sb_lds[kbl * NB + jb] = staged_scale<C>(g.sb[jblk * g.sb_j + (kb0 + kbl) * g.sb_r]);
        }
      }
    }
  };

  v4f acc[C::TM][C::TN];
#pragma unroll
  for (int a = 0; a < C::TM; ++a)
#pragma unroll
    for (int b = 0; b < C::TN; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint32_t wm0 = wm * C::WM, wn0 = wn * C::WN;

  if (kb_begin < kb_end) {
    dma_block(kb_begin, 0);
    load_scales(kb_begin, (kb_end - kb_begin) < kChunk ? (kb_end - kb_begin) : kChunk);
    wait_vmcnt<0>();
    __syncthreads();
  }
  for (int64_t kb = kb_begin; kb < kb_end; ++kb) {
    const int cur = (int)((kb - kb_begin) & 1);
    const bool more = kb + 1 < kb_end;
    // the other stage was last read in the previous block, before its barrier
    if (more) dma_block(kb + 1, cur ^ 1);

    const uint8_t* ta = tiles + cur * C::STAGE;
    const uint8_t* tb = ta + C::A_BYTES;
    const uint32_t kbl = (uint32_t)((kb - kb_begin) % kChunk);

    // B fragments (the instruction's A operand) for the wave's TN sub-tiles
    v8i bf[C::TN];
#pragma unroll
    for (int ns = 0; ns < C::TN; ++ns)
      bf[ns] = C::BT ? read_frag_bt(tb, (wn0 >> 4) + ns, lane) : read_frag(tb, wn0 + ns * 16 + l16, g4);

    // A-row scales of this lane's rows i = wm0 + ms*16 + l16 sit at
    // sa_lds[kbl][l16][wm0 / 16 + ms]
    const ST* const sa_row = sa_lds + kbl * C::BM + l16 * (C::BM / 16) + (wm0 >> 4);

    if constexpr (C::PROMOTE) {
      // scale of the B side: one value (weight block) or 4 per sub-tile (rows)
      float sbv[C::BROW ? C::TN : 1][C::BROW ? 4 : 1];
      if constexpr (C::BROW) {
#pragma unroll
        for (int ns = 0; ns < C::TN; ++ns) {
          const v4f w = *reinterpret_cast<const v4f*>(sb_lds + kbl * C::BN + wn0 + ns * 16 + g4 * 4);
#pragma unroll
          for (int t = 0; t < 4; ++t) sbv[ns][t] = w[t];
        }
      } else {
        sbv[0][0] = sb_lds[kbl * (C::BN / 128) + (wn0 >> 7)];
      }
      // One MFMA per (ms, ns) sub-tile from zero, into one of four register
      // buffers; its scaled product is added to the accumulators three
      // sub-tiles later, so that the matrix core and the vector ALU work side
      // by side and each product is read well after its MFMA has written it.
      // Row tile ms+1's A fragment and scale are read during row tile ms,
      // into one of three buffers (row ms-2's, no longer in use).
      constexpr int STEPS = C::TM * C::TN, LAG = 3;
      static_assert(C::TN >= LAG, "the lagging promotions reach back at most one row tile");
      v8i af[3];
      float sa[3];
      af[0] = read_frag(ta, wm0 + l16, g4);
      sa[0] = sa_row[0];
      v4f pp[4];
#pragma unroll
      for (int k = 0; k < STEPS + LAG; ++k) {
        if (k < STEPS) {
          const int ms = k / C::TN, ns = k % C::TN;
          if (k < LAG) mfma16_zero(pp[k & 3], bf[ns], af[ms % 3]);
          else mfma16_zero(pp[k & 3], bf[ns], af[ms % 3], pp[(k - LAG) & 3]);
          if (ns == 0 && ms + 1 < C::TM) {
            af[(ms + 1) % 3] = read_frag(ta, wm0 + (ms + 1) * 16 + l16, g4);
            sa[(ms + 1) % 3] = sa_row[ms + 1];
          }
        }
        if (k >= LAG) {
          const int j = k - LAG, ms = j / C::TN, ns = j % C::TN;
          // the block's first product: only LAG MFMAs (and no promotions)
          // were issued since its MFMA, so add the missing wait states
          if (k == LAG) asm volatile("s_nop 4" : "+v"(pp[j & 3]));
          const v4f p = pp[j & 3];
          if constexpr (C::BROW) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc[ms][ns][t] = __builtin_fmaf(p[t], sa[ms % 3] * sbv[ns][t], acc[ms][ns][t]);
          } else {
            const float sc = sa[ms % 3] * sbv[0][0];
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[ms][ns][t] = __builtin_fmaf(p[t], sc, acc[ms][ns][t]);
          }
          // an empty marker: this promotion stays ahead of the next MFMA
          asm volatile("" : "+v"(acc[ms][ns]));
        }
      }
    } else {
      // scaled MFMA: every lane passes the E8M0 byte of its own operand row
      uint32_t saw[(C::TM + 3) / 4];
#pragma unroll
      for (int w = 0; w < (C::TM + 3) / 4; ++w) saw[w] = *reinterpret_cast<const uint32_t*>(sa_row + 4 * w);
      uint32_t sbw[(C::TN + 3) / 4];
      if constexpr (C::BROW) {
#pragma unroll
        for (int w = 0; w < (C::TN + 3) / 4; ++w)
          sbw[w] = *reinterpret_cast<const uint32_t*>(sb_lds + kbl * C::BN + l16 * (C::BN / 16) + (wn0 >> 4) + 4 * w);
      } else {
        const uint32_t e = sb_lds[kbl * (C::BN / 128) + (wn0 >> 7)];
#pragma unroll
        for (int w = 0; w < (C::TN + 3) / 4; ++w) sbw[w] = e * 0x01010101u;
      }
#pragma unroll
      for (int ms = 0; ms < C::TM; ++ms) {
        const v8i af = read_frag(ta, wm0 + ms * 16 + l16, g4);
#pragma unroll
        for (int ns = 0; ns < C::TN; ++ns) {
#define FP8BLK_MFMA_SCALED(OA, OB)                                                                            \
  acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[ns], af, acc[ms][ns], 0, 0, OA,           \
                                                                  (int)sbw[ns >> 2], OB, (int)saw[ms >> 2])
          // op_sel picks the byte of the scale word; it must be a constant
          switch (((ns & 3) << 2) | (ms & 3)) {
            case 0: FP8BLK_MFMA_SCALED(0, 0); break;
            case 1: FP8BLK_MFMA_SCALED(0, 1); break;
            case 2: FP8BLK_MFMA_SCALED(0, 2); break;
            case 3: FP8BLK_MFMA_SCALED(0, 3); break;
            case 4: FP8BLK_MFMA_SCALED(1, 0); break;
            case 5: FP8BLK_MFMA_SCALED(1, 1); break;
            case 6: FP8BLK_MFMA_SCALED(1, 2); break;
            case 7: FP8BLK_MFMA_SCALED(1, 3); break;
            case 8: FP8BLK_MFMA_SCALED(2, 0); break;
            case 9: FP8BLK_MFMA_SCALED(2, 1); break;
            case 10: FP8BLK_MFMA_SCALED(2, 2); break;
            case 11: FP8BLK_MFMA_SCALED(2, 3); break;
            case 12: FP8BLK_MFMA_SCALED(3, 0); break;
            case 13: FP8BLK_MFMA_SCALED(3, 1); break;
            case 14: FP8BLK_MFMA_SCALED(3, 2); break;
            default: FP8BLK_MFMA_SCALED(3, 3); break;
          }
#undef FP8BLK_MFMA_SCALED
        }
      }
    }

    if (more && (kb + 1 - kb_begin) % kChunk == 0) {
      __syncthreads();  // everyone is done with this chunk's scales
      const int64_t rest = kb_end - (kb + 1);
      load_scales(kb + 1, rest < kChunk ? rest : kChunk);
    }
    wait_vmcnt<0>();  // this wave's loads of block kb+1 have landed
    __syncthreads();  // ... and every wave's; no wave reads stage cur any more
  }

  // ---- epilogue: lane holds out[i0+wm0+ms*16+l16][j0+wn0+ns*16+g4*4 .. +3]
#pragma unroll
  for (int ms = 0; ms < C::TM; ++ms) {
    const int64_t i = i0 + wm0 + ms * 16 + l16;
    if (i >= g.I) continue;
#pragma unroll
    for (int ns = 0; ns < C::TN; ++ns) {
      const int64_t j = j0 + wn0 + ns * 16 + g4 * 4;
      if (j >= g.J) continue;
      const v4f v = acc[ms][ns];
      if (g.splits > 1) {
        float* dst = g.ws + split * g.I * g.J + i * g.J + j;
        *reinterpret_cast<v4f*>(dst) = v;
      } else if (g.out_f32) {
        v4f* const dst = reinterpret_cast<v4f*>(static_cast<float*>(g.out) + i * g.J + j);
        if (g.accumulate) {
          const v4f o = *dst;
          *dst = v4f{o[0] + v[0], o[1] + v[1], o[2] + v[2], o[3] + v[3]};
        } else {
          *dst = v;
        }
      } else {
        uint2 o;
        o.x = bf16x2_rne(v[0], v[1]);
        o.y = bf16x2_rne(v[2], v[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + i * g.J + j) = o;
      }
    }
  }
}

// Deterministic split-K reduction: out[idx] = sum over s in order of ws[s][idx] (added to
// out[idx] when accumulating).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int splits, int64_t n4,
                                                            void* out, bool out_f32, bool accumulate) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n4; v += stride) {
    v4f s = reinterpret_cast<const v4f*>(ws)[v];
    for (int k = 1; k < splits; ++k) {
      const v4f t = reinterpret_cast<const v4f*>(ws + (int64_t)k * n4 * 4)[v];
      s[0] += t[0]; s[1] += t[1]; s[2] += t[2]; s[3] += t[3];
    }
    if (out_f32) {
      if (accumulate) {
        const v4f o = reinterpret_cast<const v4f*>(out)[v];
        s = v4f{o[0] + s[0], o[1] + s[1], o[2] + s[2], o[3] + s[3]};
      }
      reinterpret_cast<v4f*>(out)[v] = s;
    } else {
      uint2 o;
      o.x = bf16x2_rne(s[0], s[1]);
      o.y = bf16x2_rne(s[2], s[3]);
      reinterpret_cast<uint2*>(out)[v] = o;
    }
  }
}

// ------------------------------------------------------------ dispatch ----

using PromoteBlock = Cfg<256, 128, 2, 2, true, false>;
using PromoteRow = Cfg<256, 128, 2, 2, true, true>;
using ScaledBlock = Cfg<256, 128, 2, 2, false, false>;
using ScaledRow = Cfg<256, 128, 2, 2, false, true>;
using PromoteBlockBT = Cfg<256, 128, 2, 2, true, false, true>;
using ScaledBlockBT = Cfg<256, 128, 2, 2, false, false, true>;

hipError_t ensure_lds_limit(const void* kernel, int bytes, std::atomic<uint64_t>* done) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit && (done->load(std::memory_order_acquire) & bit)) return hipSuccess;
  if (hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) return e;
  if (bit) done->fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

template <class C>
static hipError_t launch_cfg(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles_m = (g.I + C::BM - 1) / C::BM;
  const int64_t tiles_n = (g.J + C::BN - 1) / C::BN;
  const int64_t nkb = g.R / 128;
  const int splits = g.splits > 0 ? g.splits : 1;
  const int64_t kb_per_split = (nkb + splits - 1) / splits;
  const int64_t blocks = tiles_m * tiles_n * splits;
  static std::atomic<uint64_t> attr_set{0};
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&gemm_kernel<C>), C::LDS, &attr_set)) return e;
  hipLaunchKernelGGL(gemm_kernel<C>, dim3((uint32_t)blocks), dim3(C::THREADS), C::LDS, stream, g, tiles_m, tiles_n,
                     kb_per_split);
  return hipGetLastError();
}

static hipError_t launch_splitk_reduce(const GemmArgs& g, hipStream_t stream) {
  const int64_t n4 = g.I * g.J / 4;
  int64_t rblocks = (n4 + 255) / 256;
  if (rblocks > 4096) rblocks = 4096;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)rblocks), dim3(256), 0, stream, g.ws, g.splits, n4, g.out,
                     g.out_f32, g.accumulate);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, GemmAlgo algo, hipStream_t stream) {
  // the 256x256 kernel needs no split-K reduction (Wgrad runs stream-K)
  if (algo == GemmAlgo::ScaledMfma && gemm_mx_eligible(g)) return launch_gemm_mx(g, stream);
  hipError_t e;
  if (g.bt)
    e = algo == GemmAlgo::Promote ? launch_cfg<PromoteBlockBT>(g, stream) : launch_cfg<ScaledBlockBT>(g, stream);
  else if (algo == GemmAlgo::Promote)
    e = g.bmode == BScale::Row ? launch_cfg<PromoteRow>(g, stream) : launch_cfg<PromoteBlock>(g, stream);
  else
    e = g.bmode == BScale::Row ? launch_cfg<ScaledRow>(g, stream) : launch_cfg<ScaledBlock>(g, stream);
  if (e != hipSuccess || g.splits <= 1) return e;
  return launch_splitk_reduce(g, stream);
}

}  // namespace fp8blk
