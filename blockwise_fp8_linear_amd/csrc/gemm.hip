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
// XOR-swizzled by (row & 7).  That leaves a two-way LDS bank conflict on the
// fragment reads (rows r and r + 8 of a 16-row fragment collide: the
// counters read about 2e7 conflict cycles per launch); a swizzle that folds
// in row >> 3 removes most of it but measured no faster, since this
// kernel's time goes elsewhere, so the simpler one stays.  One
// v_mfma_*_16x16x128_f8f6f4 consumes exactly one 128-deep block for a 16x16
// sub-tile, so the per-block scale product is applied
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
#include "fp8blk_plan.h"

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

// Output tile t of a tiles_m x tiles_n grid -> its first row and column:
// consecutive tiles walk down a group of GM tile rows before moving right,
// so that tiles in flight together share operand panels in L2.
template <class C>
__device__ __forceinline__ void gk_tile_origin(int64_t tile, int64_t tiles_m, int64_t tiles_n, int64_t& i0,
                                               int64_t& j0) {
  constexpr int64_t GM = 8;
  const int64_t group = tile / (GM * tiles_n);
  const int64_t first_m = group * GM;
  const int64_t gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int64_t in_group = tile - group * GM * tiles_n;
  i0 = (first_m + in_group % gsize) * C::BM;
  j0 = (in_group / gsize) * C::BN;
}

// The contraction of the BM x BN output tile at (i0, j0) over the 128-blocks
// [kb_begin, kb_end) into acc (zeroed first).  On return every direct load
// has landed and every wave has passed the last barrier, so the LDS may be
// refilled at once.
template <class C>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, uint8_t* lds, int64_t i0, int64_t j0, int64_t kb_begin,
                                          int64_t kb_end, v4f (&acc)[C::TM][C::TN]) {
  uint8_t* const tiles = lds;
  typedef typename C::SType ST;
  ST* const sa_lds = reinterpret_cast<ST*>(lds + 2 * C::STAGE);
  ST* const sb_lds = reinterpret_cast<ST*>(lds + 2 * C::STAGE + C::SA_BYTES);

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const uint32_t l16 = lane & 15, g4 = lane >> 4;

  const int64_t nkb = g.R / 128;
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
          // the block's last LAG products have no later MFMA to pass them
          // through, so nothing else keeps their promotions from moving up
          // to right behind their own MFMAs (a reordered build did that and
          // read a product 7 wait states after its MFMA): these wait states,
          // after the last MFMA and tied to every product buffer, pin them
          if (k == STEPS) asm volatile("s_nop 7\n\ts_nop 7" : "+v"(pp[0]), "+v"(pp[1]), "+v"(pp[2]), "+v"(pp[3]));
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
}

// Store a tile's accumulators: lane holds rows i0+wm0+ms*16+l16 and columns
// j0+wn0+ns*16+g4*4 .. +3 of a row-major rows x cols matrix (row stride ld)
// of fp32 (f32; acc: out += tile) or bf16 bits; rows and columns past the
// edge are not stored.
template <class C>
__device__ __forceinline__ void gk_store(const v4f (&acc)[C::TM][C::TN], void* out, int64_t ld, int64_t rows,
                                         int64_t cols, bool f32, bool accumulate, int64_t i0, int64_t j0) {
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t wm0 = (wave / C::WAVES_N) * C::WM, wn0 = (wave % C::WAVES_N) * C::WN;
  const uint32_t l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int ms = 0; ms < C::TM; ++ms) {
    const int64_t i = i0 + wm0 + ms * 16 + l16;
    if (i >= rows) continue;
#pragma unroll
    for (int ns = 0; ns < C::TN; ++ns) {
      const int64_t j = j0 + wn0 + ns * 16 + g4 * 4;
      if (j >= cols) continue;
      const v4f v = acc[ms][ns];
      if (f32) {
        v4f* const dst = reinterpret_cast<v4f*>(static_cast<float*>(out) + i * ld + j);
        if (accumulate) {
          const v4f o = *dst;
          *dst = v4f{o[0] + v[0], o[1] + v[1], o[2] + v[2], o[3] + v[3]};
        } else {
          *dst = v;
        }
      } else {
        uint2 o;
        o.x = bf16x2_rne(v[0], v[1]);
        o.y = bf16x2_rne(v[2], v[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + i * ld + j) = o;
      }
    }
  }
}

// One output tile per workgroup, the whole reduction (Fprop and Dgrad).
template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_kernel(GemmArgs g, int64_t tiles_m, int64_t tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int64_t i0, j0;
  gk_tile_origin<C>(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, i0, j0);
  v4f acc[C::TM][C::TN];
  gemm_tile<C>(g, lds, i0, j0, 0, g.R / 128, acc);
  gk_store<C>(acc, g.out, g.J, g.I, g.J, g.out_f32, g.accumulate, i0, j0);
}

// Wgrad (long reduction over tokens, few output tiles) on a persistent grid,
// partitioned as in the block-scaled-MFMA kernel's Wgrad (gemm_mx.hip, see
// fp8blk_plan.h): whole waves of tiles data-parallel, the rest stream-K over
// 512-deep units; a piece of a tile shared by several workgroups goes, in
// fp32, to its own slot of the workspace, and gk_fixup_kernel adds the
// pieces of every shared tile in reduction order (deterministic).  No
// workgroup waits for another.
__device__ __forceinline__ int64_t gk_start(int64_t w, int64_t W, int64_t G) { return w * W / G; }
__device__ __forceinline__ int64_t gk_owner(int64_t u, int64_t W, int64_t G) { return ((u + 1) * G - 1) / W; }
__device__ __forceinline__ int64_t gk_slot(const uint16_t* table, int64_t r, bool first) {
  const uint32_t e = table[r];
  return (int64_t)(e >> 1) + (first ? 0 : (int64_t)(e & 1));
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_sk_kernel(GemmArgs g, SkGeom sg, float* partials) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int64_t G = gridDim.x;
  const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t UB = sg.ublocks, U = g.R / (128 * UB);  // 128-blocks per unit, units per tile
  v4f acc[C::TM][C::TN];
  for (int64_t t = w; t < sg.dp_tiles; t += G) {
    int64_t i0, j0;
    gk_tile_origin<C>(t, sg.tiles_m, sg.tiles_n, i0, j0);
    gemm_tile<C>(g, lds, i0, j0, 0, U * UB, acc);
    gk_store<C>(acc, g.out, g.J, g.I, g.J, g.out_f32, g.accumulate, i0, j0);
  }
  const int64_t W = sg.units, Gs = sg.sk_grid;
  const int64_t r = sg.sk_tiles > 0 ? (w % sg.sk_tiles) * (Gs / sg.sk_tiles) + w / sg.sk_tiles : w;
  const int64_t ubeg = w < Gs ? gk_start(r, W, Gs) : 0, uend = w < Gs ? gk_start(r + 1, W, Gs) : 0;
  for (int64_t u = ubeg; u < uend;) {
    const int64_t ts = u / U;
    const int64_t lo = u - ts * U;
    const int64_t hi = (uend - ts * U) < U ? (uend - ts * U) : U;
    int64_t i0, j0;
    gk_tile_origin<C>(sg.dp_tiles + ts, sg.tiles_m, sg.tiles_n, i0, j0);
    gemm_tile<C>(g, lds, i0, j0, lo * UB, hi * UB, acc);
    if (lo == 0 && hi == U) {
      gk_store<C>(acc, g.out, g.J, g.I, g.J, g.out_f32, g.accumulate, i0, j0);
    } else {
      float* const slot = partials + gk_slot(sg.slot, r, u == ubeg) * (int64_t)(C::BM * C::BN);
      gk_store<C>(acc, slot, C::BN, C::BM, C::BN, true, false, 0, 0);
    }
    u = ts * U + hi;
  }
}

// The shared tiles of gemm_sk_kernel: block (ts, rr) sums rows
// 16 rr .. 16 rr + 15 of stream-K tile ts over its pieces in reduction order
// (piece 0: the last segment of range f, the tile's first, if f started in an
// earlier tile, else f's first segment; piece k >= 1: the first segment of
// range f + k) and stores them.
template <class C>
__global__ __launch_bounds__(256) void gk_fixup_kernel(GemmArgs g, SkGeom sg, const float* __restrict__ partials) {
  constexpr int ROWS = 16, PER = ROWS * C::BN / 4 / 256;  // float4 per thread
  static_assert(PER >= 1 && ROWS * C::BN == PER * 4 * 256, "whole float4s per thread");
  const int64_t ts = blockIdx.x / (C::BM / ROWS);
  const int64_t r0 = (blockIdx.x % (C::BM / ROWS)) * ROWS;
  const int64_t U = g.R / (128 * sg.ublocks), W = sg.units, G = sg.sk_grid;
  const int64_t f = gk_owner(ts * U, W, G);
  const int pieces = (int)(gk_owner(ts * U + U - 1, W, G) - f + 1);
  if (pieces == 1) return;  // stored by the GEMM itself
  const int64_t first_slot = gk_slot(sg.slot, f, !(gk_start(f, W, G) < ts * U));
  int64_t i0, j0;
  gk_tile_origin<C>(sg.dp_tiles + ts, sg.tiles_m, sg.tiles_n, i0, j0);
  v4f sum[PER];
  for (int pc = 0; pc < pieces; ++pc) {
    const int64_t slot = pc == 0 ? first_slot : gk_slot(sg.slot, f + pc, true);
    const v4f* src = reinterpret_cast<const v4f*>(partials + slot * (int64_t)(C::BM * C::BN) + r0 * C::BN);
    v4f v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) v[k] = __builtin_nontemporal_load(src + threadIdx.x + 256 * k);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (pc == 0) sum[k] = v[k];
      else sum[k] = v4f{sum[k][0] + v[k][0], sum[k][1] + v[k][1], sum[k][2] + v[k][2], sum[k][3] + v[k][3]};
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int64_t i = i0 + r0 + idx / (C::BN / 4), j = j0 + (idx % (C::BN / 4)) * 4;
    if (i >= g.I || j >= g.J) continue;
    if (g.out_f32) {
      v4f* const dst = reinterpret_cast<v4f*>(static_cast<float*>(g.out) + i * g.J + j);
      if (g.accumulate) {
        const v4f o = *dst;
        *dst = v4f{o[0] + sum[k][0], o[1] + sum[k][1], o[2] + sum[k][2], o[3] + sum[k][3]};
      } else {
        *dst = sum[k];
      }
    } else {
      uint2 o;
      o.x = bf16x2_rne(sum[k][0], sum[k][1]);
      o.y = bf16x2_rne(sum[k][2], sum[k][3]);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + i * g.J + j) = o;
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
  static std::atomic<uint64_t> attr_set{0};
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&gemm_kernel<C>), C::LDS, &attr_set)) return e;
  hipLaunchKernelGGL(gemm_kernel<C>, dim3((uint32_t)(tiles_m * tiles_n)), dim3(C::THREADS), C::LDS, stream, g, tiles_m,
                     tiles_n);
  return hipGetLastError();
}

// Wgrad on the general kernel: the persistent stream-K launch, then the
// fix-up of shared tiles if there are any.
template <class C>
static hipError_t launch_cfg_sk(const GemmArgs& g, hipStream_t stream) {
  const SkPlan p = general_sk_plan(g.I, g.J, g.R);
  static_assert(C::BM == kGeneralTileI && C::BN == kGeneralTileJ, "the plan's tile shape");
  static std::atomic<uint64_t> attr_set{0};
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&gemm_sk_kernel<C>), C::LDS, &attr_set)) return e;
  float* const partials = p.slots > 0 ? g.ws : nullptr;
  hipLaunchKernelGGL(gemm_sk_kernel<C>, dim3((uint32_t)p.grid), dim3(C::THREADS), C::LDS, stream, g, p.geom,
                     partials);
  if (hipError_t e = hipGetLastError()) return e;
  if (p.slots == 0) return hipSuccess;
  const int64_t sk_tiles = p.geom.tiles_m * p.geom.tiles_n - p.geom.dp_tiles;
  hipLaunchKernelGGL(gk_fixup_kernel<C>, dim3((uint32_t)(sk_tiles * (C::BM / 16))), dim3(256), 0, stream, g, p.geom,
                     partials);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, GemmAlgo algo, hipStream_t stream) {
  if (algo == GemmAlgo::ScaledMfma && gemm_mx_eligible(g)) return launch_gemm_mx(g, stream);
  if (g.bt)
    return algo == GemmAlgo::Promote ? launch_cfg<PromoteBlockBT>(g, stream) : launch_cfg<ScaledBlockBT>(g, stream);
  if (g.bmode == BScale::Row)
    return algo == GemmAlgo::Promote ? launch_cfg_sk<PromoteRow>(g, stream) : launch_cfg_sk<ScaledRow>(g, stream);
  return algo == GemmAlgo::Promote ? launch_cfg<PromoteBlock>(g, stream) : launch_cfg<ScaledBlock>(g, stream);
}

}  // namespace fp8blk
