// Host-side launch plans of libfp8blk's persistent GEMM kernels: how the
// reduction work of a contraction's output tiles is cut into ranges, one per
// workgroup, and where the partial tiles of shared output tiles go in the
// workspace.  Plain C++ (plan.cpp), shared by the kernels' launchers and by
// the C ABI layer's workspace queries.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fp8blk {

// The persistent grid: one workgroup per CU of an MI355X (fewer for tiny
// shapes).  At most this many ranges, so slot tables have this many entries.
constexpr int64_t kSkGrid = 256;
// Output tile edge of the block-scaled-MFMA kernels (gemm_mx.hip).
constexpr int64_t kMxTile = 256;
// 128-blocks of a reduction whose weight-block scales those kernels hold in
// LDS at once.
constexpr int64_t kMxMaxKb = 128;
// Output tile of the general kernel (gemm.hip).
constexpr int64_t kGeneralTileI = 256, kGeneralTileJ = 128;

// Range w of a grid of G over W units: [w W / G, (w + 1) W / G).
inline int64_t h_start(int64_t w, int64_t W, int64_t G) { return w * W / G; }
// The range that holds unit u: the largest w with start(w) <= u.
inline int64_t h_owner(int64_t u, int64_t W, int64_t G) { return ((u + 1) * G - 1) / W; }

// A workgroup's range is a run of segments, one per output tile it touches;
// only its first and last segment can cover part of a tile.  Such a partial
// tile is stored, in fp32, to a tile-sized slot of the workspace, and a
// fix-up kernel adds the pieces of every shared tile in reduction order.
// Slots are numbered densely over the partial segments, in range order:
// slot[r] = (P(r) << 1) | f(r), with P(r) the number of partial segments of
// ranges 0 .. r-1 and f(r) = 1 if range r's first segment is partial.  Range
// r's first segment (if partial) uses slot P(r), its last one (if partial
// and not also the first) P(r) + f(r).

// Wgrad alone on the persistent grid (gemm_mx_streamk_kernel, and the general
// kernel's gemm_sk_kernel): whole waves of tiles run data-parallel, the rest
// stream-K over 512-deep units.
struct SkGeom {
  int64_t tiles_m, tiles_n;
  int64_t dp_tiles;  // tiles [0, dp_tiles) are data-parallel
  int64_t units;     // W: stream-K units (of the tiles from dp_tiles on)
  int64_t sk_grid;   // Gs = min(G, W): workgroups with stream-K work
  int64_t sk_tiles;  // T' when the ranges are permuted (see gemm_mx.hip), else 0
  int64_t ublocks;   // 128-blocks per unit
  uint16_t slot[kSkGrid];
};

struct SkPlan {
  SkGeom geom;
  int64_t grid;
  int64_t slots;  // partial segments (workspace slots); 0: no tile is shared
  size_t bytes;   // workspace bytes
};

// Output tiles of tile_i x tile_j (the block-scaled-MFMA kernel's 256 x 256
// by default; the general kernel's are 256 x 128), slots of that many fp32;
// units of ublocks 128-blocks (4 by default: the reduction's block count
// must then be a multiple of 4).
SkPlan sk_plan(int64_t I, int64_t J, int64_t R, int64_t tile_i = kMxTile, int64_t tile_j = kMxTile,
               int64_t ublocks = 4);

// The general kernel's Wgrad plan: 256 x 128 tiles, units of four 128-blocks
// when the reduction allows, else of one.
SkPlan general_sk_plan(int64_t I, int64_t J, int64_t R);

// Dgrad (problem 0: I = M, J = K, R = N, weight-block scales) and Wgrad
// (problem 1: I = N, J = K, R = M, row scales) of one linear in one
// persistent launch (gemm_mx_bwd_kernel).  Both problems' tiles are cut into
// 512-deep units, problem 0's first; range r (one per workgroup) covers
// units [rstart[r], rstart[r+1]).  The host picks the ranges per shape
// (plan.cpp): one even cut of all units, or problem 0 on the first G0 ranges
// and problem 1 on the rest, each cut evenly in whole tiles or in units.
struct BwdGeom {
  int64_t tm0, tn0, u0, t0;  // problem 0: tile grid, units per tile, tiles
  int64_t tm1, tn1, u1;      // problem 1
  int64_t w0;                // units of problem 0
  int64_t units;             // W, all units
  // dealing: when problem p's tiles lie in ranges [rp0[p], rp0[p] + rpn[p])
  // alone and each of them holds whole tiles, deal[p] = 1 and the j-th tile
  // of the problem's i-th range is tile j * rpn[p] + i, so that the ranges
  // running side by side work on neighbouring tiles and share operand panels
  // in L2 (such tiles never reach the fix-up).
  int64_t rp0[2], rpn[2], deal[2];
  uint32_t rstart[kSkGrid + 1];
  uint16_t slot[kSkGrid];
  // the tiles that several ranges share (problem 0's numbered 0 .. t0 - 1,
  // then problem 1's), ascending: each range boundary inside a tile makes
  // that tile shared, so there are fewer than kSkGrid
  int64_t nshared;
  uint32_t shared[kSkGrid];
};

struct BwdPlan {
  BwdGeom geom;
  int64_t grid;
  int64_t slots;
  size_t bytes;
};

// The largest r < G with rstart[r] <= u: the range that holds unit u (ranges
// are never empty).
inline int64_t h_range_of(const uint32_t* rstart, int64_t G, int64_t u) {
  int64_t lo = 0, hi = G;
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) / 2;
    if ((int64_t)rstart[mid] <= u) lo = mid;
    else hi = mid;
  }
  return lo;
}

BwdPlan bwd_plan(int64_t M, int64_t N, int64_t K);

}  // namespace fp8blk
