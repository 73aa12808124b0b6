// Host-side launch planning of libfp8blk's GEMMs (see fp8blk_plan.h): the
// persistent kernels' range partitions and workspace slot tables (both
// GEMM kernels' stream-K Wgrad, the fused backward), workspace sizes, and
// which kernel a contraction can take.
// Plain C++, no device code, so that it can also be built and exercised on a
// host alone (the C ABI's sanitizer test does).
#include "fp8blk_plan.h"

#include "fp8blk_launch.h"

namespace fp8blk {

namespace {

constexpr size_t kSlotBytes = size_t(kMxTile) * kMxTile * sizeof(float);

// Walk range r's segments the way the kernels do -- over units [ubeg, uend)
// of one or two problems laid end to end (problem 1 starting at unit w0,
// tiles of u0 and u1 units) -- and report whether its first and its last
// segment cover only part of their tile.
void partial_ends(int64_t ubeg, int64_t uend, int64_t w0, int64_t u0, int64_t u1, bool* first, bool* last) {
  *first = *last = false;
  bool is_first = true;
  for (int64_t u = ubeg; u < uend;) {
    const bool p1 = u >= w0;
    const int64_t base = p1 ? w0 : 0, U = p1 ? u1 : u0;
    const int64_t ts = (u - base) / U;
    const int64_t lo = u - base - ts * U;
    const int64_t tend = base + (ts + 1) * U;
    const int64_t hi = (uend < tend ? uend : tend) - base - ts * U;
    const bool partial = !(lo == 0 && hi == U);
    const int64_t next = base + ts * U + hi;
    if (partial) {
      if (is_first) *first = true;
      else *last = true;  // a later partial segment can only be the range's last
    }
    is_first = false;
    u = next;
  }
}

// Fill slot[0 .. G) for ranges [rstart[r], rstart[r+1]) of units over the
// problems above; returns the number of partial segments (slots).
int64_t slot_table(uint16_t* slot, const uint32_t* rstart, int64_t G, int64_t w0, int64_t u0, int64_t u1) {
  int64_t P = 0;
  for (int64_t r = 0; r < G; ++r) {
    bool f = false, l = false;
    partial_ends(rstart[r], rstart[r + 1], w0, u0, u1, &f, &l);
    slot[r] = (uint16_t)((P << 1) | (f ? 1 : 0));
    P += (f ? 1 : 0) + (l ? 1 : 0);
  }
  for (int64_t r = G; r < kSkGrid; ++r) slot[r] = (uint16_t)(P << 1);
  return P;
}

// ---- the fused backward's partition.  Cost model, in 128-blocks of MFMA
// work: every segment pays a fixed cost (pipeline fill and epilogue, about
// eight blocks' worth on the decoder layer's shapes), a partial one a little
// more (its tile leaves in fp32), and any partial tile at all costs the
// fix-up launch that follows.
constexpr double kSegCost = 8.0, kPartialCost = 2.0, kFixupCost = 8.0;

// Makespan of explicit ranges (exact walk), fix-up included.
double ranges_cost(const uint32_t* rstart, int64_t G, int64_t w0, int64_t u0, int64_t u1) {
  double worst = 0.0;
  bool any_partial = false;
  for (int64_t r = 0; r < G; ++r) {
    double c = 0.0;
    for (int64_t u = rstart[r]; u < (int64_t)rstart[r + 1];) {
      const bool p1 = u >= w0;
      const int64_t base = p1 ? w0 : 0, U = p1 ? u1 : u0;
      const int64_t ts = (u - base) / U, lo = u - base - ts * U;
      const int64_t tend = base + (ts + 1) * U;
      const int64_t hi = ((int64_t)rstart[r + 1] < tend ? (int64_t)rstart[r + 1] : tend) - base - ts * U;
      const bool partial = !(lo == 0 && hi == U);
      c += 4.0 * (double)(hi - lo) + kSegCost + (partial ? kPartialCost : 0.0);
      any_partial = any_partial || partial;
      u = base + ts * U + hi;
    }
    worst = c > worst ? c : worst;
  }
  return worst + (any_partial ? kFixupCost : 0.0);
}

// One side of a two-sided partition: T tiles of U units on Gs ranges, cut in
// whole tiles (tile_cut) or evenly in units; estimated makespan and whether
// tiles get shared.
double side_cost(int64_t T, int64_t U, int64_t Gs, bool tile_cut, bool* partial) {
  if (tile_cut) {
    *partial = false;
    const int64_t tiles = (T + Gs - 1) / Gs;
    return (double)tiles * (4.0 * (double)U + kSegCost);
  }
  const int64_t W = T * U, q = (W + Gs - 1) / Gs;
  *partial = !(W % Gs == 0 && q % U == 0);
  const int64_t segs = (q + U - 1) / U + (*partial ? 1 : 0);
  return 4.0 * (double)q + (double)segs * kSegCost + (*partial ? 2.0 * kPartialCost : 0.0);
}

// Range starts of one side: ranges [r0, r0 + Gs) over units [base, base + T U).
// A whole-tile cut gives the first T mod Gs ranges one tile more than the
// others (so that tile j of range i can be j Gs + i).
void side_starts(uint32_t* rstart, int64_t r0, int64_t Gs, int64_t base, int64_t T, int64_t U, bool tile_cut) {
  const int64_t each = T / Gs, extra = T % Gs;
  for (int64_t i = 0; i < Gs; ++i)
    rstart[r0 + i] = (uint32_t)(base + (tile_cut ? U * (i * each + (i < extra ? i : extra)) : (i * T * U) / Gs));
}

}  // namespace

SkPlan sk_plan(int64_t I, int64_t J, int64_t R, int64_t tile_i, int64_t tile_j, int64_t ublocks) {
  SkPlan p{};
  p.geom.tiles_m = (I + tile_i - 1) / tile_i;
  p.geom.tiles_n = (J + tile_j - 1) / tile_j;
  p.geom.ublocks = ublocks;
  const int64_t T = p.geom.tiles_m * p.geom.tiles_n, U = R / (128 * ublocks);
  p.grid = T * U < kSkGrid ? T * U : kSkGrid;
  p.geom.dp_tiles = (T / p.grid) * p.grid;
  const int64_t W = (T - p.geom.dp_tiles) * U;
  const int64_t Gs = W < p.grid ? W : p.grid;
  p.geom.units = W;
  p.geom.sk_grid = Gs;
  p.geom.sk_tiles = (W > 0 && W % Gs == 0 && U % (W / Gs) == 0) ? T - p.geom.dp_tiles : 0;
  if (W > 0) {
    uint32_t rstart[kSkGrid + 1];
    for (int64_t r = 0; r <= Gs; ++r) rstart[r] = (uint32_t)h_start(r, W, Gs);
    p.slots = slot_table(p.geom.slot, rstart, Gs, W, U, U);
  } else {
    p.slots = 0;
  }
  p.bytes = (size_t)p.slots * (size_t)(tile_i * tile_j) * sizeof(float);
  return p;
}

BwdPlan bwd_plan(int64_t M, int64_t N, int64_t K) {
  BwdPlan p{};
  BwdGeom& b = p.geom;
  b.tm0 = (M + kMxTile - 1) / kMxTile;
  b.tn0 = (K + kMxTile - 1) / kMxTile;
  b.u0 = N / 512;
  b.t0 = b.tm0 * b.tn0;
  b.tm1 = (N + kMxTile - 1) / kMxTile;
  b.tn1 = (K + kMxTile - 1) / kMxTile;
  b.u1 = M / 512;
  b.w0 = b.t0 * b.u0;
  b.units = b.w0 + b.tm1 * b.tn1 * b.u1;
  const int64_t G = b.units < kSkGrid ? b.units : kSkGrid;
  const int64_t T1 = b.tm1 * b.tn1;
  p.grid = G;

  // candidate 1: one even cut of all units (the two problems end to end)
  for (int64_t r = 0; r <= G; ++r) b.rstart[r] = (uint32_t)h_start(r, b.units, G);
  double best = ranges_cost(b.rstart, G, b.w0, b.u0, b.u1), best_sum = 1e300;
  // candidates 2: problem 0 on ranges [0, G0), problem 1 on [G0, G), each side
  // cut in whole tiles or evenly in units (no side gets more ranges than it
  // has tiles or units, so no range is empty)
  int64_t best_g0 = 0;
  bool best_cut0 = false, best_cut1 = false;
  for (int64_t g0 = 1; g0 < G; ++g0) {
    const int64_t g1 = G - g0;
    for (int m = 0; m < 4; ++m) {
      const bool cut0 = m & 1, cut1 = m & 2;
      if ((cut0 ? b.t0 : b.w0) < g0 || (cut1 ? T1 : b.units - b.w0) < g1) continue;
      bool part0 = false, part1 = false;
      const double c0 = side_cost(b.t0, b.u0, g0, cut0, &part0);
      const double c1 = side_cost(T1, b.u1, g1, cut1, &part1);
      const double c = (c0 > c1 ? c0 : c1) + ((part0 || part1) ? kFixupCost : 0.0);
      // ties: the one with less work in all (more slack off the critical side)
      const double sum = (double)g0 * c0 + (double)g1 * c1;
      if (c < best - 1e-9 || (best_g0 > 0 && c < best + 1e-9 && sum < best_sum)) {
        best = c;
        best_sum = sum;
        best_g0 = g0;
        best_cut0 = cut0;
        best_cut1 = cut1;
      }
    }
  }
  if (best_g0 > 0) {
    side_starts(b.rstart, 0, best_g0, 0, b.t0, b.u0, best_cut0);
    side_starts(b.rstart, best_g0, G - best_g0, b.w0, T1, b.u1, best_cut1);
    b.rstart[G] = (uint32_t)b.units;
  }
  // dealing: a problem whose ranges are its own and hold whole tiles
  const int64_t pfirst[2] = {0, b.w0}, plast[2] = {b.w0, b.units}, pU[2] = {b.u0, b.u1};
  for (int q = 0; q < 2; ++q) {
    const int64_t r0 = h_range_of(b.rstart, G, pfirst[q]);
    const int64_t r1 = h_range_of(b.rstart, G, plast[q] - 1) + 1;
    bool whole = (int64_t)b.rstart[r0] == pfirst[q] && (int64_t)b.rstart[r1] == plast[q];
    for (int64_t r = r0; whole && r < r1; ++r)
      whole = ((int64_t)b.rstart[r] - pfirst[q]) % pU[q] == 0 && ((int64_t)b.rstart[r + 1] - pfirst[q]) % pU[q] == 0;
    // every range but the last ones holds the same number of tiles, one more
    // than those: tile j of range i is then j * R + i for all of them
    int64_t hi_count = 0, lo_count = 0;
    bool dealable = whole;
    for (int64_t r = r0; dealable && r < r1; ++r) {
      const int64_t n = ((int64_t)b.rstart[r + 1] - (int64_t)b.rstart[r]) / pU[q];
      if (r == r0) hi_count = n;
      if (n == hi_count && lo_count == 0) continue;
      if (lo_count == 0 && n == hi_count - 1) lo_count = n;
      else if (n != lo_count) dealable = false;
    }
    b.rp0[q] = r0;
    b.rpn[q] = r1 - r0;
    b.deal[q] = dealable ? 1 : 0;
  }
  p.slots = slot_table(b.slot, b.rstart, G, b.w0, b.u0, b.u1);
  p.bytes = (size_t)p.slots * kSlotBytes;
  // shared tiles: those holding a range boundary strictly inside them
  b.nshared = 0;
  for (int64_t r = 1; r < G; ++r) {
    const int64_t u = b.rstart[r];
    const bool p1 = u >= b.w0;
    const int64_t off = u - (p1 ? b.w0 : 0), U = p1 ? b.u1 : b.u0;
    if (off % U == 0) continue;  // the boundary falls between tiles
    const int64_t t = (p1 ? b.t0 : 0) + off / U;
    if (b.nshared == 0 || b.shared[b.nshared - 1] != (uint32_t)t) b.shared[b.nshared++] = (uint32_t)t;
  }
  return p;
}

bool gemm_mx_eligible(const GemmArgs& g) {
  const int64_t nkb = g.R / 128;
  if (nkb % 4 != 0) return false;
  // weight-block mode keeps the tile's whole column of block scales in LDS
  if (g.bmode == BScale::Block && nkb > kMxMaxKb) return false;
  // per-lane 32-bit offsets: 256 rows x R bytes of codes, 256 rows of scales
  // (the transposed-B layout: 128 rows x J bytes)
  if (g.R > (int64_t(1) << 22)) return false;
  if (g.bt && (g.bmode != BScale::Block || g.J > (int64_t(1) << 22))) return false;
  if ((reinterpret_cast<uintptr_t>(g.sa) & 15) != 0) return false;
  if (g.bmode == BScale::Row && (reinterpret_cast<uintptr_t>(g.sb) & 15) != 0) return false;
  return true;
}

size_t gemm_mx_workspace_bytes(int64_t I, int64_t J, int64_t R, BScale bmode) {
  if (bmode != BScale::Row || (R / 128) % 4 != 0) return 0;
  return sk_plan(I, J, R).bytes;
}

SkPlan general_sk_plan(int64_t I, int64_t J, int64_t R) {
  return sk_plan(I, J, R, kGeneralTileI, kGeneralTileJ, (R / 128) % 4 == 0 ? 4 : 1);
}

// The general kernel's Wgrad (row scales) runs stream-K on 256 x 128 tiles.
static size_t general_workspace_bytes(int64_t I, int64_t J, int64_t R, BScale bmode) {
  return bmode == BScale::Row ? general_sk_plan(I, J, R).bytes : 0;
}

size_t gemm_workspace_bytes(int64_t I, int64_t J, int64_t R, BScale bmode) {
  // enough for either path: the stream-K partial tiles of the general kernel
  // or of the block-scaled-MFMA kernel
  const size_t gen = general_workspace_bytes(I, J, R, bmode);
  const size_t mx = gemm_mx_workspace_bytes(I, J, R, bmode);
  return gen > mx ? gen : mx;
}

size_t gemm_path_workspace_bytes(const GemmArgs& g, GemmAlgo algo) {
  if (algo == GemmAlgo::ScaledMfma && gemm_mx_eligible(g))
    return g.bmode == BScale::Row ? sk_plan(g.I, g.J, g.R).bytes : 0;
  return general_workspace_bytes(g.I, g.J, g.R, g.bmode);
}

bool gemm_mx_bwd_eligible(const GemmArgs& gd, const GemmArgs& gw) {
  return gd.bmode == BScale::Block && gw.bmode == BScale::Row && gemm_mx_eligible(gd) && gemm_mx_eligible(gw) &&
         gd.I == gw.R && gd.R == gw.I && gd.J == gw.J;
}

size_t gemm_mx_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if ((N / 128) % 4 != 0 || (M / 128) % 4 != 0) return 0;
  return bwd_plan(M, N, K).bytes;
}

}  // namespace fp8blk
