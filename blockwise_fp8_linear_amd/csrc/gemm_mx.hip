// Block-scaled FP8 GEMM for gfx950 on the block-scaled MFMA -- the fast path.
//
// Same contraction as gemm.hip (out[i][j] = sum over 128-deep reduction
// blocks b of sa(i,b) * sb(j,b) * sum_r A[i][r] B[j][r]; Fprop, Dgrad and Wgrad
// of the FP8 linear layer, "Puro-2B ... part 3/7", section 3.2), built for
// throughput:
//   * 256 x 256 output tile per workgroup, 4 waves of 128 x 128, one
//     workgroup per CU (146 KiB of LDS);
//   * v_mfma_scale_f32_32x32x64_f8f6f4: each operand row carries its
//     power-of-two scale as an E8M0 byte (the fp32 scale's exponent field),
//     applied inside the matrix core; products accumulate in place, in fp32,
//     so the accumulators never leave the matrix registers;
//   * the reduction advances in 64-deep stages through two LDS "pair slots"
//     of 128-deep (one scale block) whole-cache-line rows, filled by direct
//     global->LDS 16-byte loads (no staging registers) issued between the
//     MFMAs, one pair slot in flight while the other is consumed;
//   * 16-byte chunks of a row are XOR-swizzled so that fragment reads are
//     free of bank conflicts; fragments are double-buffered in registers;
//   * the scale bytes of four consecutive 128-blocks are packed in one
//     register per operand row and picked by the instruction's op_sel; the
//     weight-block scales of a tile are staged in LDS once;
//   * the epilogue stages each wave's tile through LDS and stores whole rows
//     with non-temporal stores: measured faster than plain ones (the fused
//     backward most), although issuing them takes a little longer, so the
//     gain is outside the epilogue -- plausibly the output no longer sitting
//     dirty in L2 for operand fetches to evict (the fetch counts are the
//     same either way);
//   * Dgrad can read the weight codes W[n][k] as quantized (reduction along
//     the rows, no transposed copy): that B tile is staged as 128 weight rows
//     of 256 bytes and its fragments come from LDS transpose reads
//     (ds_read_b64_tr_b8);
//   * Wgrad (long reduction over tokens, few output tiles) runs stream-K:
//     a persistent grid in which every workgroup does the same number of
//     512-deep reduction units; a tile shared by several workgroups is
//     written piece by piece to fp32 workspace slots, which a fix-up kernel
//     adds in reduction order (deterministic; no workgroup waits for
//     another).  The fused backward (Dgrad and Wgrad of one linear in one
//     persistent launch) partitions its units the same way, by host-planned
//     ranges.
// Requirements (else the caller falls back to gemm.hip): the number of
// 128-blocks of the reduction is a multiple of 4 (at most 128 for
// weight-block scales) and the per-row scale arrays are 16-byte aligned.
#include "fp8blk_device.h"
#include "fp8blk_launch.h"
#include "fp8blk_plan.h"

namespace fp8blk {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = (int)kMxTile, BN = (int)kMxTile, BK = 64, THREADS = 256;
constexpr int WM = 128, WN = 128;          // wave tile
constexpr int TM = WM / 32, TN = WN / 32;  // 32x32 MFMA tiles per wave
// The LDS ring holds two "pair slots"; a pair slot holds two consecutive
// 64-deep stages (one 128-deep scale block) of both tiles as whole 128-byte
// rows, so every direct load reads whole cache lines.
constexpr int PK = 2 * BK;                         // bytes of a row in a pair slot
constexpr int A_SLOT = BM * PK, B_SLOT = BN * PK, SLOT = A_SLOT + B_SLOT;  // 64 KiB
constexpr int SLOTS = 2;
constexpr int SC_BYTES = 8192;            // one group of raw scales: A rows, then B rows
constexpr int MAX_KB = (int)kMxMaxKb;     // 128-blocks per segment with weight-block scales (held in LDS)
constexpr int BS_BYTES = 4 * MAX_KB * 4;  // the 4 waves' weight-block scales of a segment, fp32
constexpr int LDS_BYTES = SLOTS * SLOT + 2 * SC_BYTES + BS_BYTES;  // 146 KiB
constexpr int LOADS_A = A_SLOT / 1024 / (THREADS / 64);  // 1 KiB per wave instruction
constexpr int LOADS_B = B_SLOT / 1024 / (THREADS / 64);
constexpr int LOADS_PER_PAIR = LOADS_A + LOADS_B;          // per wave

template <int V>
struct IntC {
  static constexpr int value = V;
};

// 16-byte chunk swizzle of a 128-byte row: physical chunk = logical ^ swz(row).
// Within any 8 (or 16) consecutive rows read with one logical chunk, the
// physical chunks cover distinct banks for both 32- and 64-bank LDS.  It
// depends on row & 31 only, so it is the same for every 32-row MFMA tile.
__device__ __forceinline__ uint32_t swz(uint32_t row) { return ((row & 31) ^ ((row & 31) >> 3)) & 7; }

// The transposed-B tile (128 reduction rows x 256 bytes = 16 chunks): physical
// chunk = logical ^ swz_bt(row).  A transpose read of one 16-lane group
// touches 8 consecutive rows (aligned to 8) at one or two adjacent logical
// chunks; 2 * (row & 7) sends those 16 (row, chunk) pairs to 16 distinct
// chunk positions, i.e. distinct banks.
__device__ __forceinline__ uint32_t swz_bt(uint32_t row) { return 2 * (row & 7); }


// fp32 power-of-two scales -> E8M0 bytes (their exponent fields), 4 packed.
__device__ __forceinline__ uint32_t pack_e8(u32x4 s) {
  return ((s[0] >> 23) & 0xFF) | (((s[1] >> 23) & 0xFF) << 8) | (((s[2] >> 23) & 0xFF) << 16) |
         (((s[3] >> 23) & 0xFF) << 24);
}

// Output tile t -> its first row and column: consecutive tiles walk down a
// group of GM tile rows before moving right, so that tiles in flight
// together share operand panels in L2.  With GM = 4, the 32 tiles an XCD
// runs at once are 4 tile rows x 8 tile columns, and its 4 row panels of A
// (2 MiB at a 2048-deep reduction) stay in the XCD's 4 MiB L2 from one
// round of tiles to the next; GM = 8 measured the same at 8192 rows and 7%
// slower at 32768 rows, GM = 16 and 32 slower everywhere.
__device__ __forceinline__ void tile_origin(int64_t tile, int64_t tiles_m, int64_t tiles_n, int64_t& i0,
                                            int64_t& j0) {
  constexpr int64_t GM = 4;
  const int64_t group = tile / (GM * tiles_n);
  const int64_t first_m = group * GM;
  const int64_t gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int64_t in_group = tile - group * GM * tiles_n;
  i0 = (first_m + in_group % gsize) * BM;
  j0 = (in_group / gsize) * BN;
}

// The contraction of one output tile over the 128-blocks
// [kb_begin, kb_begin + nkb_seg) (nkb_seg a multiple of 4) into acc, which it
// zeroes first.  On return every direct load has landed; the LDS ring may
// still be read by other waves until the next barrier.
// BT: B is stored [R][J] (the weight codes W[n][k] read as quantized, for
// Dgrad) instead of [J][R]; weight-block scales only.
template <bool BROW, bool BT = false>
__device__ __forceinline__ void mma_segment(const GemmArgs& g, uint8_t* lds, int64_t i0, int64_t j0, int64_t kb_begin,
                                            int64_t nkb_seg, v16f (&acc)[TM][TN]) {
  static_assert(!(BT && BROW), "the transposed-B layout is Dgrad's, with weight-block scales");
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = lds_offset(lds);
  const uint32_t l32 = lane & 31, g2 = lane >> 5;
  const int64_t R = g.R, nkb = R / 128;
  const int ngroup = (int)(nkb_seg / 4);  // groups of four 128-blocks

  // ---- direct loads of the tiles, one pair slot (128-deep) at a time.  Wave
  // instruction u fills 8 rows x 128 B; lane p writes LDS bytes p*16..+15 of
  // that KiB: row p/8, physical chunk p%8, which holds logical chunk
  // (p%8) ^ swz(row).  Per-lane 32-bit offsets from wave-uniform bases; rows
  // past a ragged edge read the last row (valid memory, results never stored).
  const int npair = (int)nkb_seg;
  const uint8_t* baseA = g.a + i0 * R + kb_begin * 128;
  // BT: pair p is reduction rows 128 (kb_begin + p) .. +127 of B[R][J]
  const uint8_t* baseB = BT ? g.b + kb_begin * 128 * g.J + j0 : g.b + j0 * R + kb_begin * 128;
  const int64_t pairB = BT ? 128 * g.J : PK;  // bytes from one pair of B to the next
  uint32_t offLA[LOADS_A], offLB[LOADS_B];
#pragma unroll
  for (int u = 0; u < LOADS_A; ++u) {
    const uint32_t row = (wave * LOADS_A + u) * 8 + (lane >> 3);
    int64_t gr = i0 + row;
    gr = gr < g.I ? gr : g.I - 1;
    offLA[u] = (uint32_t)((gr - i0) * R) + (((lane & 7) ^ swz(row)) << 4);
  }
#pragma unroll
  for (int u = 0; u < LOADS_B; ++u) {
    if constexpr (BT) {
      // wave instruction u fills 4 reduction rows x 256 B: lane p writes
      // row p/16, physical chunk p%16, which holds logical chunk
      // (p%16) ^ swz_bt(row), i.e. columns j0 + 16 * logical ..; chunks
      // past a ragged column edge read the last valid one (never stored)
      const uint32_t row = (wave * LOADS_B + u) * 4 + (lane >> 4);
      int64_t col = 16 * (int64_t)((lane & 15) ^ swz_bt(row));
      col = j0 + col < g.J - 16 ? col : g.J - 16 - j0;
      offLB[u] = (uint32_t)(row * g.J + col);
    } else {
      const uint32_t row = (wave * LOADS_B + u) * 8 + (lane >> 3);
      int64_t gr = j0 + row;
      gr = gr < g.J ? gr : g.J - 1;
      offLB[u] = (uint32_t)((gr - j0) * R) + (((lane & 7) ^ swz(row)) << 4);
    }
  }
  // pair p -> slot p % SLOTS; a pair past the end reloads the last one into a
  // slot that is never read again (keeps the waits uniform).
  // issue_one(p, u): the wave's u-th direct load of pair p (u < LOADS_A: A).
  auto issue_one = [&](int pr, int u) {
    const int pc = pr < npair ? pr : npair - 1;
    const uint32_t slot = lds0 + (uint32_t)(pr % SLOTS) * SLOT;
    if (u < LOADS_A)
      dma16(baseA + (int64_t)pc * PK, offLA[u], slot + (wave * LOADS_A + u) * 1024);
    else
      dma16(baseB + (int64_t)pc * pairB, offLB[u - LOADS_A], slot + A_SLOT + (wave * LOADS_B + u - LOADS_A) * 1024);
  };
  auto issue_pair = [&](int pr) {
#pragma unroll
    for (int u = 0; u < LOADS_PER_PAIR; ++u) issue_one(pr, u);
  };

  // ---- direct loads of the raw fp32 scales of a group (four 128-blocks):
  // lane of wave w handles operand row 64w + lane, 16 bytes (blocks kb..kb+3).
  // Double buffered in LDS behind the tile ring.
  uint8_t* const sc_lds = lds + SLOTS * SLOT;
  // byte offsets of this lane's scale row from the tile's first row, block kb_begin
  uint32_t offSA, offSB = 0;
  const uint8_t* baseSA = reinterpret_cast<const uint8_t*>(g.sa + i0 * nkb + kb_begin);
  const uint8_t* baseSB = reinterpret_cast<const uint8_t*>(g.sb + j0 * nkb + kb_begin);
  {
    int64_t r = i0 + wave * 64 + lane;
    r = r < g.I ? r : g.I - 1;
    offSA = (uint32_t)((r - i0) * nkb * 4);
  }
  if constexpr (BROW) {
    int64_t r = j0 + wave * 64 + lane;
    r = r < g.J ? r : g.J - 1;
    offSB = (uint32_t)((r - j0) * nkb * 4);
  }
  const uint32_t sc0 = lds0 + SLOTS * SLOT;
  auto issue_scales = [&](int q) {  // group q -> scale buffer q & 1
    const int qc = q < ngroup ? q : ngroup - 1;
    const uint32_t buf = sc0 + (uint32_t)(q & 1) * SC_BYTES;
    dma16(baseSA + 16 * qc, offSA, buf + wave * 1024);
    if constexpr (BROW) dma16(baseSB + 16 * qc, offSB, buf + 4096 + wave * 1024);
  };

  // ---- fragment reads: lane l holds row l%32 of a 32-row MFMA tile and, of
  // stage s (half s%2 of its pair slot), logical chunks 4*(s%2) + 2*(l/32) and
  // the next one (A and B use the same K order).
  const uint32_t wm0 = wm * WM, wn0 = wn * WN;
  const uint32_t swzl = swz(l32);
  const uint32_t cA0 = (((0 + 2 * g2) ^ swzl) << 4), cA1 = (((4 + 2 * g2) ^ swzl) << 4);
  const uint32_t rowA = (wm0 + l32) * PK, rowB = A_SLOT + (wn0 + l32) * PK;
  // the second chunk sits 16 bytes after or before the first (signed!)
  const int32_t hiOff = ((swzl & 1) ? -16 : 16);
  auto read_frag = [&](int st, uint32_t off) {
    const uint8_t* p = lds + ((st >> 1) % SLOTS) * SLOT + off + ((st & 1) ? cA1 : cA0);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p + hiOff);
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // BT: the fragment of the wave's t-th 32-column tile in four transpose
  // reads.  Lane l needs column wn0 + 32t + l%32 and, of stage st, reduction
  // values 32 (l/32) .. +31 (the same order as A's fragment); read r covers
  // 8r .. 8r+7 of them.  In the lane's 16-lane group q = l/16 and position
  // s = l%16 it addresses row 64 (st%2) + 32 (q/2) + 8r + s/2 of the pair at
  // columns wn0 + 32t + 16 (q%2) + 8 (s%2) .. +7; swz_bt(row) = 2 (s/2).
  const uint32_t bt_q = lane >> 4, bt_s = lane & 15;
  const uint32_t bt_row = (32 * (bt_q >> 1) + (bt_s >> 1)) * 256 + 8 * (bt_s & 1);
  auto read_frag_bt = [&](int st, int t) {
    const uint8_t* p = lds + ((st >> 1) % SLOTS) * SLOT + A_SLOT + bt_row + (st & 1) * 64 * 256 +
                       (((((wn0 >> 4) + 2 * t + (bt_q & 1)) ^ (2 * (bt_s >> 1))) << 4));
    v8i f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const v2i_t v = lds_read_tr8(p + r * 8 * 256);
      f[2 * r] = v[0];
      f[2 * r + 1] = v[1];
    }
    return f;
  };
  auto read_frag_b = [&](int st, int t) {
    if constexpr (BT) return read_frag_bt(st, t);
    else return read_frag(st, rowB + t * 32 * PK);
  };
  auto read_frags = [&](int st, v8i* fa, v8i* fb) {
#pragma unroll
    for (int t = 0; t < TM; ++t) fa[t] = read_frag(st, rowA + t * 32 * PK);
#pragma unroll
    for (int t = 0; t < TN; ++t) fb[t] = read_frag_b(st, t);
  };
  // packed E8M0 scale bytes of group q for this lane's operand rows
  // (row wm0 + 32t + l%32 of A, of B in row mode); weight-block scales are
  // uniform over the wave's 128 columns (clamped on a ragged edge, where the
  // columns are computed but not stored).
  const int64_t jblk = ((j0 + wn0) >> 7) < (g.J >> 7) ? ((j0 + wn0) >> 7) : (g.J >> 7) - 1;
  // weight-block mode: every scale this wave needs (its block column, all
  // nkb_seg <= MAX_KB blocks of the segment) is loaded once, up front, into
  // LDS -- no scalar loads in the main loop (their shared lgkmcnt would make
  // the LDS waits drain them)
  constexpr uint32_t bs_area = SLOTS * SLOT + 2 * SC_BYTES;
  auto issue_block_scales = [&]() {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(g.sb + jblk * g.sb_j + kb_begin * g.sb_r);
#pragma unroll
    for (int h = 0; h < MAX_KB / 64; ++h) {
      int64_t k = h * 64 + lane;
      k = k < nkb_seg ? k : nkb_seg - 1;
      dma4(base, (uint32_t)(k * g.sb_r * 4), lds0 + bs_area + wave * (MAX_KB * 4) + h * 256);
    }
  };
  auto read_scales = [&](int q, uint32_t* pa, uint32_t* pb) {
    const uint8_t* buf = sc_lds + (q & 1) * SC_BYTES;
#pragma unroll
    for (int t = 0; t < TM; ++t) pa[t] = pack_e8(*reinterpret_cast<const u32x4*>(buf + (wm0 + t * 32 + l32) * 16));
    if constexpr (BROW) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
        pb[t] = pack_e8(*reinterpret_cast<const u32x4*>(buf + 4096 + (wn0 + t * 32 + l32) * 16));
    } else {
      // this wave's weight block, blocks 4q..4q+3 of the slice (same
      // address in every lane: a broadcast read)
      const int qc = q < ngroup ? q : ngroup - 1;
      const uint32_t e = pack_e8(*reinterpret_cast<const u32x4*>(lds + bs_area + wave * (MAX_KB * 4) + 16 * qc));
#pragma unroll
      for (int t = 0; t < TN; ++t) pb[t] = e;
    }
  };

#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = v16f{};

  uint32_t sa_cur[TM], sb_cur[TN];
  v8i fa[2][TM], fb[2][TN];

  // prologue: every weight-block scale of the segment, the scales of group 0,
  // pairs 0 and 1; then pair 0 and group 0 visible
  if constexpr (!BROW) issue_block_scales();
  issue_scales(0);
  issue_pair(0);
  issue_pair(1);
  wait_vmcnt<LOADS_PER_PAIR>();  // everything but pair 1 has landed
  lds_barrier();
  read_frags(0, fa[0], fb[0]);
  read_scales(0, sa_cur, sb_cur);

  // One 64-deep stage s.  Entry: stage s's fragments are in registers (set
  // BUF).  The 16 MFMAs of stage s are issued in pairs; between pairs the wave
  // reads one fragment of stage s+1 (into the other register set).  An odd
  // stage s = 2p-1 first waits for pair p (stage s+1's slot, issued two stages
  // ago), passes a barrier -- after which no wave reads the slot of pair p-1
  // any more (stage s's fragments were read during stage s-1) -- and refills
  // that slot with pair p+1, two direct loads per MFMA pair.  Even stages
  // need no wait and no barrier: stage s+1 is in the same pair.  The
  // sched_barrier fences pin the interleaving.
  static_assert(TM == 4 && TN == 4 && LOADS_PER_PAIR == 16, "one read + two loads per MFMA pair");
  auto stage_step = [&](int st, auto buf_tag, auto opsel_tag) {
    constexpr int OPSEL = decltype(opsel_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;  // also the parity of st
    constexpr int NXT = BUF ^ 1;
    if constexpr (BUF == 1) {
      wait_vmcnt<0>();  // this wave's part of pair (st+1)/2 (and older) has landed
      lds_barrier();    // ... and every wave's
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int a = p >> 1, b0 = 2 * (p & 1);
      acc[a][b0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[BUF][b0], fa[BUF][a], acc[a][b0], 0, 0, OPSEL,
                                                                   (int)sb_cur[b0], OPSEL, (int)sa_cur[a]);
      acc[a][b0 + 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          fb[BUF][b0 + 1], fa[BUF][a], acc[a][b0 + 1], 0, 0, OPSEL, (int)sb_cur[b0 + 1], OPSEL, (int)sa_cur[a]);
      // next stage's fragments in the order its MFMAs consume them
      if (p == 0) fa[NXT][0] = read_frag(st + 1, rowA);
      else if (p <= 4) fb[NXT][p - 1] = read_frag_b(st + 1, p - 1);
      else fa[NXT][p - 4] = read_frag(st + 1, rowA + (p - 4) * 32 * PK);
      if constexpr (BUF == 1) {
        issue_one((st + 3) >> 1, 2 * p);
        issue_one((st + 3) >> 1, 2 * p + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One loop iteration = one group = four 128-blocks = eight 64-deep stages;
  // op_sel (the byte of the packed scales) is a constant in each step.
  for (int q = 0; q < ngroup; ++q) {
    const int st = 8 * q;
    issue_scales(q + 1);  // buffer (q+1)&1 was last read at the end of group q-2
    stage_step(st + 0, IntC<0>{}, IntC<0>{});
    stage_step(st + 1, IntC<1>{}, IntC<0>{});
    stage_step(st + 2, IntC<0>{}, IntC<1>{});
    stage_step(st + 3, IntC<1>{}, IntC<1>{});
    stage_step(st + 4, IntC<0>{}, IntC<2>{});
    stage_step(st + 5, IntC<1>{}, IntC<2>{});
    stage_step(st + 6, IntC<0>{}, IntC<3>{});
    stage_step(st + 7, IntC<1>{}, IntC<3>{});
    // group q+1's scales were issued before the waits of this group's odd
    // stages and every wave passed their barriers
    read_scales(q + 1, sa_cur, sb_cur);
  }
  wait_vmcnt<0>();  // no direct load may still target this workgroup's LDS at exit
}

// Where a tile goes: a row-major matrix (bf16 bits or fp32) of rows x cols,
// row stride ld elements; rows and columns past the edge are not stored.
struct Dst {
  void* out;
  int64_t ld, rows, cols;
  bool f32;
  bool acc;  // fp32: out += tile
};

// Store a finished 256 x 256 tile at (i0, j0) of d.  src(a, b) yields the
// wave's 32x32 accumulator tile (a, b) in the MFMA register layout; it is
// called once per tile, in (a, b) order.  Starts with a barrier, so the LDS
// ring and any earlier staging are free.
template <int BATCH, class Src>
__device__ __forceinline__ void store_tile_from(const Dst& d, uint8_t* lds, int64_t i0, int64_t j0, Src src) {
  // ---- epilogue, staged through LDS so that global stores are whole rows,
  // non-temporal (the output is not read again here; see the file header).
  // src(a, b) lane l, element e holds row i = wm0 + 32a + l%32 and column
  // j = wn0 + 32b + 8*(e/4) + 4*(l/32) + e%4.  Each wave writes its 128 x 128
  // tile to its own 32 KiB of LDS in units of 4 consecutive columns, the unit
  // index XOR-swizzled by (row & 31) (conflict-free: the 32 lanes of a write
  // hit 32 different units of their rows), then reads back 16-byte pieces of
  // whole rows and stores them coalesced.  fp32 output goes in two halves of
  // 64 rows.
  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const uint32_t l32 = lane & 31, g2 = lane >> 5;
  lds_barrier();  // every wave is done reading the tile ring
  {
    uint8_t* stage_area = lds + wave * 32768;
    const bool f32 = d.f32;
    float* const outf = static_cast<float*>(d.out);
    uint16_t* const outh = static_cast<uint16_t*>(d.out);
    const int64_t col0 = j0 + wn0;
    // the wave's 128 columns are all in or all out (N is a multiple of 128);
    // full: no row of the wave's tile is past the edge either
    const bool col_ok = col0 < d.cols;
    const bool full = col_ok && i0 + wm0 + WM <= d.rows;
    if (!f32) {
      // bf16: unit = 8 bytes, row = 256 bytes, all 128 rows at once
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const v16f v = src(a, b);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t row = a * 32 + l32;
            const uint32_t unit = (8 * b + 2 * q + g2) ^ (row & 31);
            uint2 o;
            o.x = bf16x2_rne(v[4 * q], v[4 * q + 1]);
            o.y = bf16x2_rne(v[4 * q + 2], v[4 * q + 3]);
            *reinterpret_cast<uint2*>(stage_area + row * 256 + unit * 8) = o;
          }
        }
      // read: 16 lanes per row (16 bytes = units 2k, 2k+1 each), 4 rows per
      // pass, in batches of passes whose LDS reads are all issued before
      // the first store (a read waited for right before its own store
      // exposes the LDS latency 32 times)
#pragma unroll 1
      for (int pb = 0; pb < 32; pb += BATCH) {
        u32x4 v[BATCH];
#pragma unroll
        for (int s = 0; s < BATCH; ++s) {
          const uint32_t row = (pb + s) * 4 + (lane >> 4), k = lane & 15;
          const uint32_t pu = (2 * k) ^ (row & 31);  // physical unit of logical unit 2k
          v[s] = *reinterpret_cast<const u32x4*>(stage_area + row * 256 + (pu & ~1u) * 8);
        }
#pragma unroll
        for (int s = 0; s < BATCH; ++s) {
          const uint32_t row = (pb + s) * 4 + (lane >> 4), k = lane & 15;
          // the pair is stored swapped when its physical unit is odd (row odd)
          const u32x4 o = (row & 1) ? u32x4{v[s][2], v[s][3], v[s][0], v[s][1]} : v[s];
          const int64_t i = i0 + wm0 + row;
          if (full || (i < d.rows && col_ok))
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(outh + i * d.ld + col0 + 8 * k));
        }
      }
    } else {
      // fp32: unit = 16 bytes, row = 512 bytes, two halves of 64 rows
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
          const int a = 2 * h + a2;
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            const v16f t = src(a, b);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t row = a2 * 32 + l32;
              const uint32_t unit = (8 * b + 2 * q + g2) ^ (row & 31);
              const v4f v = {t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
              *reinterpret_cast<v4f*>(stage_area + row * 512 + unit * 16) = v;
            }
          }
        }
        // read: 32 lanes per row (one unit each), 2 rows per pass, batched
        // as above
#pragma unroll 1
        for (int pb = 0; pb < 32; pb += BATCH) {
          v4f v[BATCH];
#pragma unroll
          for (int s = 0; s < BATCH; ++s) {
            const uint32_t row = (pb + s) * 2 + (lane >> 5), k = lane & 31;
            v[s] = *reinterpret_cast<const v4f*>(stage_area + row * 512 + ((k ^ (row & 31)) * 16));
          }
          if (d.acc) {
            v4f o[BATCH];
#pragma unroll
            for (int s = 0; s < BATCH; ++s) {
              const uint32_t row = (pb + s) * 2 + (lane >> 5), k = lane & 31;
              const int64_t i = i0 + wm0 + 64 * h + row;
              if (full || (i < d.rows && col_ok)) o[s] = *reinterpret_cast<const v4f*>(outf + i * d.ld + col0 + 4 * k);
            }
#pragma unroll
            for (int s = 0; s < BATCH; ++s) {
              const uint32_t row = (pb + s) * 2 + (lane >> 5), k = lane & 31;
              const int64_t i = i0 + wm0 + 64 * h + row;
              if (full || (i < d.rows && col_ok))
                __builtin_nontemporal_store(
                    v4f{o[s][0] + v[s][0], o[s][1] + v[s][1], o[s][2] + v[s][2], o[s][3] + v[s][3]},
                    reinterpret_cast<v4f*>(outf + i * d.ld + col0 + 4 * k));
            }
          } else {
#pragma unroll
            for (int s = 0; s < BATCH; ++s) {
              const uint32_t row = (pb + s) * 2 + (lane >> 5), k = lane & 31;
              const int64_t i = i0 + wm0 + 64 * h + row;
              if (full || (i < d.rows && col_ok))
                __builtin_nontemporal_store(v[s], reinterpret_cast<v4f*>(outf + i * d.ld + col0 + 4 * k));
            }
          }
        }
      }
    }
  }
}

// Store a tile from registers.  (A local copy: reading the caller's array
// through the reference while storing to LDS makes the compiler keep it in
// memory -- hundreds of spilled registers.)
template <int BATCH>
__device__ __forceinline__ void store_tile(const Dst& d, uint8_t* lds, int64_t i0, int64_t j0,
                                           const v16f (&acc_in)[TM][TN]) {
  v16f acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = acc_in[a][b];
  store_tile_from<BATCH>(d, lds, i0, j0, [&](int a, int b) { return acc[a][b]; });
}

// One output tile per workgroup, the whole reduction (Fprop and Dgrad; BT:
// Dgrad from the weight codes as quantized).
template <bool BROW, bool BT = false>
__global__ __launch_bounds__(THREADS) void gemm_mx_kernel(GemmArgs g, int64_t tiles_m, int64_t tiles_n) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
  int64_t i0, j0;
  tile_origin(tile, tiles_m, tiles_n, i0, j0);
  v16f acc[TM][TN];
  mma_segment<BROW, BT>(g, lds, i0, j0, 0, g.R / 128, acc);
  store_tile<8>(Dst{g.out, g.J, g.I, g.J, g.out_f32, g.accumulate}, lds, i0, j0, acc);
}

// Wgrad (long reduction over tokens, few output tiles) on a persistent grid
// of G workgroups.  Whole waves of tiles are data-parallel: workgroup w
// takes tiles w, w + G, ... below dp_tiles = G * floor(T / G).  The
// remaining tiles run stream-K: their reductions are cut into units of four
// 128-blocks and workgroup w < Gs = min(G, W) takes units
// [w W / Gs, (w + 1) W / Gs) of the W = (T - dp_tiles) * U of them, in tile
// order, so every such workgroup does the same work.  When every tile splits
// into p equal ranges (Gs divides W, the range length divides U), workgroup
// w takes range (w mod T') p + w div T' of the T' stream-K tiles instead:
// the workgroups of one XCD (consecutive w) then cover different tiles at
// the same depth, sharing operand panels in L2, as a split-K launch would.
// A stream-K range is a run of segments: whole tiles are stored directly; a
// piece of a tile shared by several workgroups is stored, in fp32, to a
// tile-sized slot of the workspace (numbered densely over the partial
// segments, see fp8blk_plan.h) and a second kernel adds the pieces of every
// shared tile in reduction order (deterministic) and stores it.  No
// workgroup ever waits for another.
__device__ __forceinline__ int64_t sk_start(int64_t w, int64_t W, int64_t G) { return w * W / G; }
// the workgroup whose range holds unit u: the largest w with start(w) <= u
__device__ __forceinline__ int64_t sk_owner(int64_t u, int64_t W, int64_t G) { return ((u + 1) * G - 1) / W; }

// The slot of range r's first (first = true) or last partial segment.
__device__ __forceinline__ int64_t slot_of(const uint16_t* table, int64_t r, bool first) {
  const uint32_t e = table[r];
  return (int64_t)(e >> 1) + (first ? 0 : (int64_t)(e & 1));
}

template <bool BROW>
__global__ __launch_bounds__(THREADS) void gemm_mx_streamk_kernel(GemmArgs g, SkGeom sg, float* partials) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int64_t G = gridDim.x;
  const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t U = g.R / 512;  // units per tile
  const Dst out{g.out, g.J, g.I, g.J, g.out_f32, g.accumulate};
  v16f acc[TM][TN];
  for (int64_t t = w; t < sg.dp_tiles; t += G) {
    int64_t i0, j0;
    tile_origin(t, sg.tiles_m, sg.tiles_n, i0, j0);
    lds_barrier();  // the previous tile's epilogue is done with LDS
    mma_segment<BROW>(g, lds, i0, j0, 0, U * 4, acc);
    store_tile<1>(out, lds, i0, j0, acc);
  }
  const int64_t W = sg.units, Gs = sg.sk_grid;
  // r: this workgroup's range (and slot pair) index
  const int64_t r = sg.sk_tiles > 0 ? (w % sg.sk_tiles) * (Gs / sg.sk_tiles) + w / sg.sk_tiles : w;
  const int64_t ubeg = w < Gs ? sk_start(r, W, Gs) : 0, uend = w < Gs ? sk_start(r + 1, W, Gs) : 0;
  for (int64_t u = ubeg; u < uend;) {
    const int64_t ts = u / U;                                    // stream-K tile index
    const int64_t lo = u - ts * U;                               // first unit of the segment, within the tile
    const int64_t hi = (uend - ts * U) < U ? (uend - ts * U) : U;  // one past its last
    int64_t i0, j0;
    tile_origin(sg.dp_tiles + ts, sg.tiles_m, sg.tiles_n, i0, j0);
    lds_barrier();
    mma_segment<BROW>(g, lds, i0, j0, lo * 4, (hi - lo) * 4, acc);
    if (lo == 0 && hi == U) {
      store_tile<1>(out, lds, i0, j0, acc);
    } else {
      float* const slot = partials + slot_of(sg.slot, r, u == ubeg) * (int64_t)(BM * BN);
      store_tile<1>(Dst{slot, BN, BM, BN, true, false}, lds, 0, 0, acc);
    }
    u = ts * U + hi;
  }
}

// The shared stream-K tiles: block (ts, r) sums rows 16r..16r+15 of
// stream-K tile ts over its pieces in reduction order and stores them.
// Piece 0 is the last segment of range f (the tile's first) if f started in
// an earlier tile, else f's first segment; piece k >= 1 is the first
// segment of range f + k.
constexpr int FIX_ROWS = 16;

__global__ __launch_bounds__(256) void sk_fixup_kernel(GemmArgs g, SkGeom sg, const float* __restrict__ partials) {
  const int64_t ts = blockIdx.x / (BM / FIX_ROWS);
  const int64_t r0 = (blockIdx.x % (BM / FIX_ROWS)) * FIX_ROWS;
  const int64_t U = g.R / 512, W = sg.units, G = sg.sk_grid;
  const int64_t f = sk_owner(ts * U, W, G);
  const int pieces = (int)(sk_owner(ts * U + U - 1, W, G) - f + 1);
  if (pieces == 1) return;  // stored by the GEMM itself
  const int64_t first_slot = slot_of(sg.slot, f, !(sk_start(f, W, G) < ts * U));
  int64_t i0, j0;
  tile_origin(sg.dp_tiles + ts, sg.tiles_m, sg.tiles_n, i0, j0);
  constexpr int PER = FIX_ROWS * BN / 4 / 256;  // float4 per thread
  v4f sum[PER];
  for (int pc = 0; pc < pieces; ++pc) {
    const int64_t slot = pc == 0 ? first_slot : slot_of(sg.slot, f + pc, true);
    const v4f* src = reinterpret_cast<const v4f*>(partials + slot * (int64_t)(BM * BN) + r0 * BN);
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
    const int64_t i = i0 + r0 + idx / (BN / 4), j = j0 + (idx % (BN / 4)) * 4;
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

// ---------------------------------------------------------------------------
// Dgrad and Wgrad of one linear in one persistent stream-K launch.  Problem
// 0 is Dgrad (weight-block scales), problem 1 Wgrad (row scales); the two
// have the same FLOP count.  The reductions of all their tiles are cut into
// units of four 128-blocks, problem 0's tiles first, and range r of G takes
// units [rstart[r], rstart[r + 1]) of them: the host picks the cut that
// balances the ranges' modelled cost, tiles and partial segments both
// counted, so the CUs stay busy across both GEMMs.  Segments, slots and the
// fix-up of shared tiles work as in the Wgrad kernel above; when a problem's
// tiles fall whole into ranges of its own (dealt), the j-th tile of its i-th
// range is tile j R + i (R ranges), so that the ranges running side by side
// work on neighbouring tiles and share operand panels in L2.

// BT: Dgrad reads the weight codes as quantized (gd.b is W[N][K]).
template <bool BT>
__global__ __launch_bounds__(THREADS) void gemm_mx_bwd_kernel(GemmArgs gd, GemmArgs gw, BwdGeom bg,
                                                              float* partials) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int64_t r = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t ubeg = bg.rstart[r], uend = bg.rstart[r + 1];
  v16f acc[TM][TN];
  for (int64_t u = ubeg; u < uend;) {
    const bool p1 = u >= bg.w0;
    const int64_t base = p1 ? bg.w0 : 0, U = p1 ? bg.u1 : bg.u0;
    const int64_t ts = (u - base) / U;                     // tile of the problem, in range order
    const int64_t lo = u - base - ts * U;                   // first unit of the segment, within the tile
    const int64_t tend = base + (ts + 1) * U;
    const int64_t hi = (uend < tend ? uend : tend) - base - ts * U;  // one past its last
    const int q = p1 ? 1 : 0;
    // dealt: the j-th tile of the problem's i-th range is tile j * R + i
    const int64_t tt = bg.deal[q] ? ((u - ubeg) / U) * bg.rpn[q] + (r - bg.rp0[q]) : ts;  // the tile itself
    int64_t i0, j0;
    tile_origin(tt, p1 ? bg.tm1 : bg.tm0, p1 ? bg.tn1 : bg.tn0, i0, j0);
    lds_barrier();  // the previous segment's epilogue is done with LDS
    if (p1)
      mma_segment<true>(gw, lds, i0, j0, lo * 4, (hi - lo) * 4, acc);
    else
      mma_segment<false, BT>(gd, lds, i0, j0, lo * 4, (hi - lo) * 4, acc);
    if (lo == 0 && hi == U) {
      const Dst d{p1 ? gw.out : gd.out, p1 ? gw.J : gd.J, p1 ? gw.I : gd.I, p1 ? gw.J : gd.J,
                  p1 ? gw.out_f32 : gd.out_f32, p1 ? gw.accumulate : gd.accumulate};
      store_tile<1>(d, lds, i0, j0, acc);
    } else {
      float* const slot = partials + slot_of(bg.slot, r, u == ubeg) * (int64_t)(BM * BN);
      store_tile<1>(Dst{slot, BN, BM, BN, true, false}, lds, 0, 0, acc);
    }
    u = base + ts * U + hi;
  }
}

// The range of a backward launch that holds unit u: the largest r < G with
// rstart[r] <= u (ranges are never empty).
__device__ __forceinline__ int64_t bwd_range_of(const BwdGeom& bg, int64_t G, int64_t u) {
  int64_t lo = 0, hi = G;
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) / 2;
    if ((int64_t)bg.rstart[mid] <= u) lo = mid;
    else hi = mid;
  }
  return lo;
}

// The shared tiles of a backward launch: block (k, r) sums rows
// 16r..16r+15 of the k-th shared tile t = shared[k] (problem 0's tiles
// numbered first, then problem 1's) over its pieces in reduction order and
// stores them; slots as in sk_fixup_kernel.  (Tiles of a dealt problem are
// never shared.)
__global__ __launch_bounds__(256) void bwd_fixup_kernel(GemmArgs gd, GemmArgs gw, BwdGeom bg, int64_t G,
                                                        const float* __restrict__ partials) {
  const int64_t t = bg.shared[blockIdx.x / (BM / FIX_ROWS)];
  const int64_t r0 = (blockIdx.x % (BM / FIX_ROWS)) * FIX_ROWS;
  const bool p1 = t >= bg.t0;
  const int64_t ts = p1 ? t - bg.t0 : t, U = p1 ? bg.u1 : bg.u0;
  const int64_t first = (p1 ? bg.w0 : 0) + ts * U;
  const int64_t f = bwd_range_of(bg, G, first);
  const int pieces = (int)(bwd_range_of(bg, G, first + U - 1) - f + 1);
  if (pieces == 1) return;  // stored by the GEMM itself
  const int64_t first_slot = slot_of(bg.slot, f, !((int64_t)bg.rstart[f] < first));
  int64_t i0, j0;
  tile_origin(ts, p1 ? bg.tm1 : bg.tm0, p1 ? bg.tn1 : bg.tn0, i0, j0);
  const int64_t I = p1 ? gw.I : gd.I, J = p1 ? gw.J : gd.J;
  void* const out = p1 ? gw.out : gd.out;
  const bool out_f32 = p1 ? gw.out_f32 : gd.out_f32, accumulate = p1 ? gw.accumulate : gd.accumulate;
  constexpr int PER = FIX_ROWS * BN / 4 / 256;  // float4 per thread
  v4f sum[PER];
  for (int pc = 0; pc < pieces; ++pc) {
    const int64_t slot = pc == 0 ? first_slot : slot_of(bg.slot, f + pc, true);
    const v4f* src = reinterpret_cast<const v4f*>(partials + slot * (int64_t)(BM * BN) + r0 * BN);
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
    const int64_t i = i0 + r0 + idx / (BN / 4), j = j0 + (idx % (BN / 4)) * 4;
    if (i >= I || j >= J) continue;
    if (out_f32) {
      v4f* const dst = reinterpret_cast<v4f*>(static_cast<float*>(out) + i * J + j);
      if (accumulate) {
        const v4f o = *dst;
        *dst = v4f{o[0] + sum[k][0], o[1] + sum[k][1], o[2] + sum[k][2], o[3] + sum[k][3]};
      } else {
        *dst = sum[k];
      }
    } else {
      uint2 o;
      o.x = bf16x2_rne(sum[k][0], sum[k][1]);
      o.y = bf16x2_rne(sum[k][2], sum[k][3]);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + i * J + j) = o;
    }
  }
}

template <class K>
hipError_t set_lds_attr(K* kernel, std::atomic<uint64_t>* done) {
  return ensure_lds_limit(reinterpret_cast<const void*>(kernel), LDS_BYTES, done);
}

template <bool BROW, bool BT>
hipError_t launch_mx(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles_m = (g.I + BM - 1) / BM;
  const int64_t tiles_n = (g.J + BN - 1) / BN;
  static std::atomic<uint64_t> attr_set{0};
  if (hipError_t e = set_lds_attr(&gemm_mx_kernel<BROW, BT>, &attr_set)) return e;
  hipLaunchKernelGGL((gemm_mx_kernel<BROW, BT>), dim3((uint32_t)(tiles_m * tiles_n)), dim3(THREADS), LDS_BYTES, stream,
                     g, tiles_m, tiles_n);
  return hipGetLastError();
}

template <bool BROW>
hipError_t launch_mx_streamk(const GemmArgs& g, hipStream_t stream) {
  const SkPlan p = sk_plan(g.I, g.J, g.R);
  static std::atomic<uint64_t> attr_set{0};
  if (hipError_t e = set_lds_attr(&gemm_mx_streamk_kernel<BROW>, &attr_set)) return e;
  float* const partials = p.slots > 0 ? g.ws : nullptr;
  hipLaunchKernelGGL(gemm_mx_streamk_kernel<BROW>, dim3((uint32_t)p.grid), dim3(THREADS), LDS_BYTES, stream, g, p.geom,
                     partials);
  if (hipError_t e = hipGetLastError()) return e;
  if (p.slots == 0) return hipSuccess;
  const int64_t sk_tiles = p.geom.tiles_m * p.geom.tiles_n - p.geom.dp_tiles;
  hipLaunchKernelGGL(sk_fixup_kernel, dim3((uint32_t)(sk_tiles * (BM / FIX_ROWS))), dim3(256), 0, stream, g, p.geom,
                     partials);
  return hipGetLastError();
}

template <bool BT>
hipError_t launch_bwd(const GemmArgs& gd, const GemmArgs& gw, float* ws, hipStream_t stream) {
  const BwdPlan p = bwd_plan(gd.I, gd.R, gd.J);
  static std::atomic<uint64_t> attr_set{0};
  if (hipError_t e = set_lds_attr(&gemm_mx_bwd_kernel<BT>, &attr_set)) return e;
  float* const partials = p.slots > 0 ? ws : nullptr;
  hipLaunchKernelGGL(gemm_mx_bwd_kernel<BT>, dim3((uint32_t)p.grid), dim3(THREADS), LDS_BYTES, stream, gd, gw, p.geom,
                     partials);
  if (hipError_t e = hipGetLastError()) return e;
  if (p.geom.nshared == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_fixup_kernel, dim3((uint32_t)(p.geom.nshared * (BM / FIX_ROWS))), dim3(256), 0, stream, gd,
                     gw, p.geom, p.grid, partials);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const GemmArgs& g, hipStream_t stream) {
  if (g.bmode == BScale::Row) return launch_mx_streamk<true>(g, stream);
  return g.bt ? launch_mx<false, true>(g, stream) : launch_mx<false, false>(g, stream);
}

hipError_t launch_gemm_mx_bwd(const GemmArgs& gd, const GemmArgs& gw, hipStream_t stream) {
  return gd.bt ? launch_bwd<true>(gd, gw, gw.ws, stream) : launch_bwd<false>(gd, gw, gw.ws, stream);
}

}  // namespace fp8blk
