// Host-side launch planning of libfp8blk's GEMMs (see fp8blk_plan.h): the
// persistent kernels' range partitions and workspace slot tables, the
// general kernel's split-K factor, and which kernel a contraction can take.
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

// Fill slot[0 .. G) for ranges of W units over the problems above; returns
// the number of partial segments (slots).
int64_t slot_table(uint16_t* slot, int64_t G, int64_t W, int64_t w0, int64_t u0, int64_t u1) {
  int64_t P = 0;
  for (int64_t r = 0; r < G; ++r) {
    bool f = false, l = false;
    partial_ends(h_start(r, W, G), h_start(r + 1, W, G), w0, u0, u1, &f, &l);
    slot[r] = (uint16_t)((P << 1) | (f ? 1 : 0));
    P += (f ? 1 : 0) + (l ? 1 : 0);
  }
  for (int64_t r = G; r < kSkGrid; ++r) slot[r] = (uint16_t)(P << 1);
  return P;
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
  p.slots = W > 0 ? slot_table(p.geom.slot, Gs, W, W, U, U) : 0;
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
  p.grid = b.units < kSkGrid ? b.units : kSkGrid;
  // round-robin tiles for a problem whose ranges all hold whole tiles: every
  // range of the grid holds the same number q of units (G divides W), the
  // problem starts and ends on range boundaries, and U divides q
  if (b.units % p.grid == 0) {
    const int64_t q = b.units / p.grid;
    if (b.w0 % q == 0 && q % b.u0 == 0) b.k0 = q / b.u0;
    if ((b.units - b.w0) % q == 0 && q % b.u1 == 0) b.k1 = q / b.u1;
  }
  p.slots = slot_table(b.slot, p.grid, b.units, b.w0, b.u0, b.u1);
  p.bytes = (size_t)p.slots * kSlotBytes;
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
