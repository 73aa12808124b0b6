// Quantizer kernels for gfx950: bf16 -> E4M3 codes + fp32 scales.
//
// What is computed ("Puro-2B ... part 3/7", section 3.2, second and third
// paragraphs): activations and gradients carry a scale for every 128-element
// run along K (the contraction's K), weights one per 128x128 tile;
// each scale a power of two (Pow2Scale), or, as a numerics variant, the
// unconstrained fp32 amax / 448 of the DeepSeek-V3 recipe that the same
// paragraph sets against it (Fp32Scale).  The scale rules and the cast are
// the readings stated in include/fp8blk.h; every kernel is instantiated for
// both rules.
//
// All three kernels are bound by HBM bandwidth (about 3 bytes moved per
// element for 0.1 flop), so the design work is in the memory access pattern:
// 16-byte loads, full 128-byte lines per store instruction where the layout
// allows, and enough independent loads in flight per wave.  The amax is an
// exact integer max over the bf16 magnitude bits, reduced across lanes with
// DPP; the scale exponent comes from the amax bits with integer ops.
#include "fp8blk_device.h"
#include "fp8blk_launch.h"

namespace fp8blk {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Row groups.  A DPP row (16 lanes) owns one 128-element group: each lane
// loads 8 bf16 (16 B), the row's 16 lanes cover the group's 256 B.  A wave
// handles 4 groups per step and kRowUnroll steps, all loads issued first.
// ---------------------------------------------------------------------------
constexpr int kRowUnroll = 4;
constexpr int kRowThreads = 256;
constexpr int kGroupsPerWave = 4 * kRowUnroll;

template <class S>
__global__ __launch_bounds__(kRowThreads) void quant_rowgroup_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ q, int64_t ld_q,
    float* __restrict__ s, uint32_t groups_per_row, uint32_t total_groups) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t sub = lane >> 4;   // which of the wave's 4 groups in a step
  const uint32_t l16 = lane & 15;   // 16-byte chunk within the group
  const uint32_t wave = blockIdx.x * (kRowThreads / 64) + (threadIdx.x >> 6);
  const uint32_t g0 = wave * kGroupsPerWave;

  u32x4 v[kRowUnroll];
  uint32_t row[kRowUnroll], col[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    uint32_t g = g0 + u * 4 + sub;
    bool ok = g < total_groups;
    uint32_t gg = ok ? g : 0;
    row[u] = gg / groups_per_row;
    col[u] = gg - row[u] * groups_per_row;
    const u32x4* p = reinterpret_cast<const u32x4*>(x + (int64_t)row[u] * ld_x + col[u] * 128 + l16 * 8);
    v[u] = ok ? __builtin_nontemporal_load(p) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    uint32_t g = g0 + u * 4 + sub;
    uint32_t m = pk_max_u16(pk_max_u16(abs2(v[u].x), abs2(v[u].y)), pk_max_u16(abs2(v[u].z), abs2(v[u].w)));
    m = max(m & 0xFFFFu, m >> 16);
    m = row16_max(m);
    const S sc(m);
    uint2 out;
    out.x = quant4(v[u].x, v[u].y, sc);
    out.y = quant4(v[u].z, v[u].w, sc);
    if (g < total_groups) {
      *reinterpret_cast<uint2*>(q + (int64_t)row[u] * ld_q + col[u] * 128 + l16 * 8) = out;
      if (l16 == 0) s[(int64_t)row[u] * groups_per_row + col[u]] = sc.s;
    }
  }
}

// ---------------------------------------------------------------------------
// Column groups (groups of 128 consecutive rows of one column, written
// transposed).  A workgroup takes a 128-row x 64-column tile: coalesced
// 16-byte row loads into LDS, then each thread owns two adjacent columns
// over 16 consecutive rows.  The 8 threads sharing a column pair reduce the
// amax with DPP and each writes 16 codes, so a column's 128 codes leave as
// one contiguous 128-byte line of qT.
// LDS tile: 128 rows x 32 words (column pairs), the word index XOR-swizzled
// by ((row / 16) & 3) * 8 so the column-pair reads hit distinct banks.
// ---------------------------------------------------------------------------
constexpr int kColTileRows = 128;
constexpr int kColTileCols = 64;
constexpr int kColThreads = 256;

__device__ __forceinline__ uint32_t col_swz(uint32_t r) { return ((r >> 4) & 3) << 3; }

template <class S>
__global__ __launch_bounds__(kColThreads) void quant_colgroup_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ qT, int64_t ld_qT,
    float* __restrict__ sT, uint32_t row_tiles, uint32_t col_tiles) {
  __shared__ uint32_t tile[kColTileRows * 32];
  const uint32_t t = threadIdx.x;
  const uint32_t logical = xcd_remap(blockIdx.x, row_tiles * col_tiles);
  const uint32_t ct = logical / row_tiles;   // consecutive logical ids walk down the rows
  const uint32_t rt = logical - ct * row_tiles;
  const int64_t m0 = (int64_t)rt * kColTileRows;
  const int64_t c0 = (int64_t)ct * kColTileCols;

  // load: 8 threads per row (16 B = 4 column pairs each), 32 rows per pass
  {
    const uint32_t chunk = t & 7;
    const uint32_t r0 = t >> 3;
    u32x4 v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t r = r0 + 32 * p;
      v[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (m0 + r) * ld_x + c0 + chunk * 8));
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t r = r0 + 32 * p;
      *reinterpret_cast<u32x4*>(&tile[r * 32 + ((chunk * 4) ^ col_swz(r))]) = v[p];
    }
  }
  __syncthreads();

  const uint32_t lane = t & 63;
  const uint32_t rp = lane & 7;                       // row part: rows rp*16 .. +15
  const uint32_t cp = (t >> 6) * 8 + (lane >> 3);     // column pair 0..31
  uint32_t w[16];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t r = rp * 16 + i;
    w[i] = tile[r * 32 + (cp ^ col_swz(r))];
    m = pk_max_u16(m, abs2(w[i]));
  }
  m = lane8_max_pk(m);
  const S inv0(m & 0xFFFFu), inv1(m >> 16);
  u32x4 o0, o1;
  o0.x = quant4_col<0>(w[0], w[1], w[2], w[3], inv0);
  o0.y = quant4_col<0>(w[4], w[5], w[6], w[7], inv0);
  o0.z = quant4_col<0>(w[8], w[9], w[10], w[11], inv0);
  o0.w = quant4_col<0>(w[12], w[13], w[14], w[15], inv0);
  o1.x = quant4_col<1>(w[0], w[1], w[2], w[3], inv1);
  o1.y = quant4_col<1>(w[4], w[5], w[6], w[7], inv1);
  o1.z = quant4_col<1>(w[8], w[9], w[10], w[11], inv1);
  o1.w = quant4_col<1>(w[12], w[13], w[14], w[15], inv1);
  const int64_t c = c0 + 2 * cp;
  *reinterpret_cast<u32x4*>(qT + c * ld_qT + m0 + rp * 16) = o0;
  *reinterpret_cast<u32x4*>(qT + (c + 1) * ld_qT + m0 + rp * 16) = o1;
  if (rp == 0) {
    const int64_t G = (int64_t)row_tiles;  // rows / 128 groups per column
    sT[c * G + rt] = inv0.s;
    sT[(c + 1) * G + rt] = inv1.s;
  }
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks.  One workgroup per block, 256 threads: thread
// (rg, cg) owns rows rg*8 .. +7 and columns cg*8 .. +7 (one 16-byte load per
// row).  The block amax is reduced over the wave with DPP/shuffles and over
// the 4 waves through LDS.  Row-major codes leave 8 bytes per lane (16 lanes
// = one 128-byte line per row); the optional transposed copy is built in
// registers with byte permutes (8x8 per thread) and leaves 8 bytes per lane.
// ---------------------------------------------------------------------------
constexpr int kBlkThreads = 256;

// Block `logical` (row-major over the row_blocks x col_blocks blocks) of one
// weight.
template <class S>
__device__ __forceinline__ void quant_block_one(const uint16_t* __restrict__ w, int64_t ld_w, uint8_t* __restrict__ q,
                                                uint8_t* __restrict__ qT, float* __restrict__ s, int64_t rows,
                                                int64_t cols, uint32_t col_blocks, uint32_t logical) {
  __shared__ uint32_t red[kBlkThreads / 64];
  const uint32_t t = threadIdx.x;
  const uint32_t bi = logical / col_blocks;
  const uint32_t bj = logical - bi * col_blocks;
  const uint32_t cg = t & 15;
  const uint32_t rg = t >> 4;                 // 0..15
  const int64_t r0 = (int64_t)bi * 128 + rg * 8;
  const int64_t cc0 = (int64_t)bj * 128 + cg * 8;

  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w + (r0 + i) * ld_w + cc0));
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    m = pk_max_u16(m, pk_max_u16(pk_max_u16(abs2(v[i].x), abs2(v[i].y)), pk_max_u16(abs2(v[i].z), abs2(v[i].w))));
  m = max(m & 0xFFFFu, m >> 16);
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  const S inv(m);

  uint32_t lo[8], hi[8];  // codes of row i: columns 0..3 in lo[i], 4..7 in hi[i]
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo[i] = quant4(v[i].x, v[i].y, inv);
    hi[i] = quant4(v[i].z, v[i].w, inv);
    *reinterpret_cast<uint2*>(q + (r0 + i) * cols + cc0) = make_uint2(lo[i], hi[i]);
  }
  if (qT != nullptr) {
    uint32_t a[4], b[4];
    // columns 0..3: rows 0..3 then rows 4..7
    transpose4x4(&lo[0], a);
    transpose4x4(&lo[4], b);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<uint2*>(qT + (cc0 + c) * rows + r0) = make_uint2(a[c], b[c]);
    transpose4x4(&hi[0], a);
    transpose4x4(&hi[4], b);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<uint2*>(qT + (cc0 + 4 + c) * rows + r0) = make_uint2(a[c], b[c]);
  }
  if (t == 0) s[(int64_t)bi * col_blocks + bj] = inv.s;
}

template <class S>
__global__ __launch_bounds__(kBlkThreads) void quant_block_kernel(
    const uint16_t* __restrict__ w, int64_t ld_w, uint8_t* __restrict__ q, uint8_t* __restrict__ qT,
    float* __restrict__ s, int64_t rows, int64_t cols, uint32_t row_blocks, uint32_t col_blocks) {
  quant_block_one<S>(w, ld_w, q, qT, s, rows, cols, col_blocks, xcd_remap(blockIdx.x, row_blocks * col_blocks));
}

// Several weights in one launch: workgroup b quantizes block b - first[j] of
// job j, the last job with first[j] <= b.
struct BlockJobs {
  BlockJob job[kMaxBlockJobs];
  uint32_t first[kMaxBlockJobs];
  int n;
};

template <class S>
__global__ __launch_bounds__(kBlkThreads) void quant_block_batch_kernel(BlockJobs jobs) {
  int j = 0;
  for (int k = 1; k < jobs.n; ++k)
    if (blockIdx.x >= jobs.first[k]) j = k;
  const BlockJob& b = jobs.job[j];
  quant_block_one<S>(b.w, b.ld_w, b.q, b.qT, b.s, b.rows, b.cols, (uint32_t)(b.cols / 128), blockIdx.x - jobs.first[j]);
}

// ---------------------------------------------------------------------------
// Row groups and column groups of the same tensor in one pass.  The pages
// keep the quantized input for Wgrad ("Puro-2B ... part 3/7", section 3.2,
// fourth paragraph); producing both orientations from one read of the bf16
// tensor saves a whole second read.  Results are identical to
// quant_rowgroup_kernel + quant_colgroup_kernel.
// A workgroup takes a 128 x 128 tile; thread t owns rows 8*(t/16) .. +7 and
// columns 8*(t%16) .. +7 (one 16-byte load per row; 16 lanes = a 256-byte
// row).  Row groups: the 16 lanes of a DPP row share the rows, so the row
// amax is a DPP reduction and each lane stores 8 codes per row.  Column
// groups: a packed per-column max over the thread's rows, then over the 16
// row blocks (wave shuffles, then LDS across the 4 waves); the thread's 8x8
// codes are formed column by column (each pair of rows gathered into one
// word by a byte permute, then converted) and staged in LDS, from where
// whole 128-byte lines of the transposed output are stored.
// ---------------------------------------------------------------------------
constexpr int kDualThreads = 256;

// Tile order of the one-pass quantizer.  A tile's scales are 128 four-byte
// values strided through s (one per row) and 128 through sT (one per
// column); the 8 tiles side by side along a row band fill one 32-byte
// sector of s, the 8 above one another one of sT.  Where the shape allows
// (kDualBlocked: a multiple of 16 row tiles and of 8 column tiles, whole
// multiples of 8 blocks), the tiles go in blocks of 8 column tiles x 16 row
// tiles, block k to the workgroups k, k + 8, ... mod 8, i.e. to one XCD
// (workgroups are dealt to the 8 XCDs in turn), walked down each column of
// the block: every sector of s and sT is then written by one XCD, whose L2
// merges the pieces before writing the sector back.  Measured on the
// activation shapes: written bytes at the algorithmic count (+11% in row-band
// order, from partial sectors written back from several L2s), and 0-8%
// faster.  Other shapes walk row band by row band.  The codes leave with
// plain stores: non-temporal ones were faster for the quantizer timed alone
// (launch after launch) but slower in a training step, where the GEMMs read
// the codes right after (they no longer found them in the caches) and the
// quantizer itself ran slower too.
constexpr uint32_t kDualBlockCols = 8, kDualBlockRows = 16;

__host__ __device__ __forceinline__ bool dual_blocked(uint32_t row_tiles, uint32_t col_tiles) {
  return row_tiles % kDualBlockRows == 0 && col_tiles % kDualBlockCols == 0 &&
         (row_tiles / kDualBlockRows) * (col_tiles / kDualBlockCols) % 8 == 0;
}

template <class S>
__global__ __launch_bounds__(kDualThreads) void quant_dual_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ s,
    uint8_t* __restrict__ qT, int64_t ld_qT, float* __restrict__ sT, uint32_t row_tiles, uint32_t col_tiles,
    uint32_t blocked) {
  __shared__ uint32_t red[kDualThreads / 64][16][4];
  __shared__ __attribute__((aligned(16))) uint2 tq[128][16];  // column codes: [column][8-row block]
  const uint32_t t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t rt, ct;
  if (blocked) {
    constexpr uint32_t kPerBlock = kDualBlockCols * kDualBlockRows;
    const uint32_t xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    const uint32_t blk = xcd + 8 * (j / kPerBlock), w = j % kPerBlock;
    const uint32_t col_blocks = col_tiles / kDualBlockCols;
    rt = (blk / col_blocks) * kDualBlockRows + w % kDualBlockRows;
    ct = (blk % col_blocks) * kDualBlockCols + w / kDualBlockRows;
  } else {
    // consecutive workgroups walk along the rows, so that the ones in flight
    // together read whole rows of x
    rt = blockIdx.x / col_tiles;
    ct = blockIdx.x - rt * col_tiles;
  }
  const int64_t m0 = (int64_t)rt * 128, c0 = (int64_t)ct * 128;
  const uint32_t rb = t >> 4, cb = t & 15;
  const int64_t r0 = m0 + rb * 8;

  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (r0 + i) * ld_x + c0 + cb * 8));

  // ---- row groups (this tile's 128 columns are exactly one group per row)
  const uint32_t G = col_tiles;  // groups per row
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t m = pk_max_u16(pk_max_u16(abs2(v[i].x), abs2(v[i].y)), pk_max_u16(abs2(v[i].z), abs2(v[i].w)));
    m = max(m & 0xFFFFu, m >> 16);
    m = row16_max(m);
    const S sc(m);
    uint2 o;
    o.x = quant4(v[i].x, v[i].y, sc);
    o.y = quant4(v[i].z, v[i].w, sc);
    uint2* const qp = reinterpret_cast<uint2*>(q + (r0 + i) * ld_q + c0 + cb * 8);
    *qp = o;
    if (cb == 0) s[(r0 + i) * G + ct] = sc.s;
  }

  // ---- column groups: packed (two columns per word) max over the 128 rows
  uint32_t cm[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    cm[0] = pk_max_u16(cm[0], abs2(v[i].x));
    cm[1] = pk_max_u16(cm[1], abs2(v[i].y));
    cm[2] = pk_max_u16(cm[2], abs2(v[i].z));
    cm[3] = pk_max_u16(cm[3], abs2(v[i].w));
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {  // the wave's 4 row blocks of this column block: lanes cb, cb+16, +32, +48
    cm[w] = pk_max_u16(cm[w], (uint32_t)__shfl_xor((int)cm[w], 16, 64));
    cm[w] = pk_max_u16(cm[w], (uint32_t)__shfl_xor((int)cm[w], 32, 64));
  }
  if (lane < 16) {
#pragma unroll
    for (int w = 0; w < 4; ++w) red[wave][cb][w] = cm[w];
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 4; ++w)
    cm[w] = pk_max_u16(pk_max_u16(red[0][cb][w], red[1][cb][w]), pk_max_u16(red[2][cb][w], red[3][cb][w]));
  // column j's amax is half j % 2 of cm[j / 2]
  const S inv[8] = {S(cm[0] & 0xFFFFu), S(cm[0] >> 16), S(cm[1] & 0xFFFFu), S(cm[1] >> 16),
                    S(cm[2] & 0xFFFFu), S(cm[2] >> 16), S(cm[3] & 0xFFFFu), S(cm[3] >> 16)};
  // The thread's 8x8 codes, one column at a time (rows 0..3 and 4..7 of
  // column j, each with the column's scale: word j / 2 of each row, half
  // j % 2), go through LDS as tq[column][row block], the 8-byte unit
  // XOR-swizzled by the column block cb, and leave as whole 128-byte lines of
  // qT: 8 lanes per column, 16 bytes (two row blocks) each.
  const int64_t cc = c0 + cb * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = j >> 1;
    uint32_t a, b;
    if (j & 1) {
      a = quant4_col<1>(v[0][m], v[1][m], v[2][m], v[3][m], inv[j]);
      b = quant4_col<1>(v[4][m], v[5][m], v[6][m], v[7][m], inv[j]);
    } else {
      a = quant4_col<0>(v[0][m], v[1][m], v[2][m], v[3][m], inv[j]);
      b = quant4_col<0>(v[4][m], v[5][m], v[6][m], v[7][m], inv[j]);
    }
    tq[cb * 8 + j][rb ^ cb] = make_uint2(a, b);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t c = k * 32 + (t >> 3), p = t & 7;
    const uint32_t pu = (2 * p) ^ (c >> 3);  // physical unit of row block 2p
    u32x4 w = *reinterpret_cast<const u32x4*>(&tq[c][pu & ~1u]);
    if (pu & 1) w = u32x4{w[2], w[3], w[0], w[1]};  // the pair is stored swapped
    u32x4* const qTp = reinterpret_cast<u32x4*>(qT + (c0 + c) * ld_qT + m0 + 16 * p);
    *qTp = w;
  }
  if (rb == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sT[(cc + j) * row_tiles + rt] = inv[j].s;
  }
}

// ------------------------------------------------------------- launchers ---

hipError_t launch_quant_rowgroup(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                 int64_t ld_q, float* s, bool fp32_scale, hipStream_t stream) {
  const uint32_t gpr = (uint32_t)(cols / 128);
  const uint32_t total = (uint32_t)(rows * gpr);
  const uint32_t waves = (total + kGroupsPerWave - 1) / kGroupsPerWave;
  const uint32_t blocks = (waves + (kRowThreads / 64) - 1) / (kRowThreads / 64);
  if (fp32_scale)
    hipLaunchKernelGGL(quant_rowgroup_kernel<Fp32Scale>, dim3(blocks), dim3(kRowThreads), 0, stream, x, ld_x, q, ld_q,
                       s, gpr, total);
  else
    hipLaunchKernelGGL(quant_rowgroup_kernel<Pow2Scale>, dim3(blocks), dim3(kRowThreads), 0, stream, x, ld_x, q, ld_q,
                       s, gpr, total);
  return hipGetLastError();
}

hipError_t launch_quant_colgroup(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qT,
                                 int64_t ld_qT, float* sT, bool fp32_scale, hipStream_t stream) {
  const uint32_t rt = (uint32_t)(rows / kColTileRows);
  const uint32_t ct = (uint32_t)(cols / kColTileCols);
  if (fp32_scale)
    hipLaunchKernelGGL(quant_colgroup_kernel<Fp32Scale>, dim3(rt * ct), dim3(kColThreads), 0, stream, x, ld_x, qT,
                       ld_qT, sT, rt, ct);
  else
    hipLaunchKernelGGL(quant_colgroup_kernel<Pow2Scale>, dim3(rt * ct), dim3(kColThreads), 0, stream, x, ld_x, qT,
                       ld_qT, sT, rt, ct);
  return hipGetLastError();
}

hipError_t launch_quant_block_batch(const BlockJob* job, int n, bool fp32_scale, hipStream_t stream) {
  BlockJobs jobs{};
  uint32_t total = 0;
  for (int k = 0; k < n; ++k) {
    jobs.job[k] = job[k];
    jobs.first[k] = total;
    total += (uint32_t)((job[k].rows / 128) * (job[k].cols / 128));
  }
  jobs.n = n;
  if (fp32_scale)
    hipLaunchKernelGGL(quant_block_batch_kernel<Fp32Scale>, dim3(total), dim3(kBlkThreads), 0, stream, jobs);
  else
    hipLaunchKernelGGL(quant_block_batch_kernel<Pow2Scale>, dim3(total), dim3(kBlkThreads), 0, stream, jobs);
  return hipGetLastError();
}

hipError_t launch_quant_block(const uint16_t* w, int64_t rows, int64_t cols, int64_t ld_w, uint8_t* q, uint8_t* qT,
                              float* s, bool fp32_scale, hipStream_t stream) {
  const uint32_t rb = (uint32_t)(rows / 128);
  const uint32_t cb = (uint32_t)(cols / 128);
  if (fp32_scale)
    hipLaunchKernelGGL(quant_block_kernel<Fp32Scale>, dim3(rb * cb), dim3(kBlkThreads), 0, stream, w, ld_w, q, qT, s,
                       rows, cols, rb, cb);
  else
    hipLaunchKernelGGL(quant_block_kernel<Pow2Scale>, dim3(rb * cb), dim3(kBlkThreads), 0, stream, w, ld_w, q, qT, s,
                       rows, cols, rb, cb);
  return hipGetLastError();
}

hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                             float* s, uint8_t* qT, int64_t ld_qT, float* sT, bool fp32_scale, hipStream_t stream) {
  const uint32_t rt = (uint32_t)(rows / 128);
  const uint32_t ct = (uint32_t)(cols / 128);
  const uint32_t blocked = dual_blocked(rt, ct) ? 1u : 0u;
  const dim3 grid(rt * ct), block(kDualThreads);
  if (fp32_scale)
    hipLaunchKernelGGL(quant_dual_kernel<Fp32Scale>, grid, block, 0, stream, x, ld_x, q, ld_q, s, qT, ld_qT, sT, rt, ct,
                       blocked);
  else
    hipLaunchKernelGGL(quant_dual_kernel<Pow2Scale>, grid, block, 0, stream, x, ld_x, q, ld_q, s, qT, ld_qT, sT, rt, ct,
                       blocked);
  return hipGetLastError();
}

}  // namespace fp8blk
