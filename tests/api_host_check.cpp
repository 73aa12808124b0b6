// Host-only check of the C ABI layer (api.cpp) and the launch planning
// (plan.cpp), built with g++ under the address and undefined-behaviour
// sanitizers (tests/test_api_sanitize.py).  The kernel launchers and the two
// HIP device queries the ABI layer makes are replaced by stubs that record
// what would have been launched, so that every entry point can be driven on
// a machine without a GPU:
//   * every argument error returns its documented status and launches
//     nothing;
//   * valid calls launch exactly the expected kernels with the expected
//     arguments (contraction extents, scale layout, algorithm);
//   * the persistent kernels' workspace slot tables agree with the segment
//     walk and the fix-up's piece enumeration the kernels perform (mirrored
//     here from gemm_mx.hip): every partial segment gets its own slot below
//     the plan's slot count, and every piece the fix-up reads is the slot its
//     producer wrote.
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <set>
#include <string>
#include <vector>

#include "../include/fp8blk.h"
#include "../blockwise_fp8_linear_amd/csrc/fp8blk_launch.h"
#include "../blockwise_fp8_linear_amd/csrc/fp8blk_plan.h"

// ---------------------------------------------------------------- stubs ----

extern "C" hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int) {
  std::memset(prop, 0, sizeof *prop);
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}

namespace {
struct Launch {
  std::string kind;
  fp8blk::GemmArgs g{}, g2{};
  int algo = -1;
  bool fp32_scale = false;
  int64_t a = 0, b = 0, c = 0;
};
std::vector<Launch> g_log;
}  // namespace

namespace fp8blk {
hipError_t launch_quant_rowgroup(const uint16_t*, int64_t rows, int64_t cols, int64_t, uint8_t*, int64_t, float*,
                                 bool f, hipStream_t) {
  g_log.push_back({"rowgroup", {}, {}, -1, f, rows, cols, 0});
  return hipSuccess;
}
hipError_t launch_quant_colgroup(const uint16_t*, int64_t rows, int64_t cols, int64_t, uint8_t*, int64_t, float*,
                                 bool f, hipStream_t) {
  g_log.push_back({"colgroup", {}, {}, -1, f, rows, cols, 0});
  return hipSuccess;
}
hipError_t launch_quant_dual(const uint16_t*, int64_t rows, int64_t cols, int64_t, uint8_t*, int64_t, float*, uint8_t*,
                             int64_t, float*, bool f, hipStream_t) {
  g_log.push_back({"dual", {}, {}, -1, f, rows, cols, 0});
  return hipSuccess;
}
hipError_t launch_quant_block_batch(const BlockJob*, int n, bool f, hipStream_t) {
  g_log.push_back({"block_batch", {}, {}, -1, f, n, 0, 0});
  return hipSuccess;
}
hipError_t launch_quant_block(const uint16_t*, int64_t rows, int64_t cols, int64_t, uint8_t*, uint8_t* qT, float*,
                              bool f, hipStream_t) {
  g_log.push_back({"block", {}, {}, -1, f, rows, cols, qT != nullptr});
  return hipSuccess;
}
hipError_t launch_gemm(const GemmArgs& g, GemmAlgo algo, hipStream_t) {
  Launch l{"gemm", g, {}, (int)algo, false, 0, 0, 0};
  g_log.push_back(l);
  return hipSuccess;
}
hipError_t launch_gemm_mx(const GemmArgs& g, hipStream_t) {
  g_log.push_back({"gemm_mx", g, {}, -1, false, 0, 0, 0});
  return hipSuccess;
}
hipError_t launch_gemm_mx_bwd(const GemmArgs& gd, const GemmArgs& gw, hipStream_t) {
  g_log.push_back({"gemm_mx_bwd", gd, gw, -1, false, 0, 0, 0});
  return hipSuccess;
}
// a stand-in address for the static scratch (never dereferenced)
alignas(256) static unsigned char g_fake_scratch[256];
hipError_t static_scratch(void** ptr, size_t* bytes) {
  *ptr = g_fake_scratch;
  *bytes = FP8BLK_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}
}  // namespace fp8blk

// ---------------------------------------------------------------- checks ---

static int g_fail = 0;
#define CHECK(cond, ...)                              \
  do {                                                \
    if (!(cond)) {                                    \
      std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
      std::printf(__VA_ARGS__);                       \
      std::printf("\n");                              \
      ++g_fail;                                       \
    }                                                 \
  } while (0)

// A heap buffer per operand, exactly sized, 16-byte aligned (the library
// never dereferences them: the stubs take their place).
struct Buf {
  std::vector<unsigned char> mem;
  unsigned char* p;
  explicit Buf(size_t n) : mem(n + 16) { p = mem.data() + ((16 - (reinterpret_cast<uintptr_t>(mem.data()) & 15)) & 15); }
};

static void expect_status(const char* what, int got, int want, size_t launches) {
  CHECK(got == want, "%s: status %d, expected %d", what, got, want);
  if (want != FP8BLK_OK) CHECK(g_log.size() == launches, "%s: an error call launched something", what);
}

static void quantizer_checks() {
  Buf x(4096 * 2), q(4096), s(64), qT(4096), sT(64);
  auto* xp = reinterpret_cast<const uint16_t*>(x.p);
  auto* sp = reinterpret_cast<float*>(s.p);
  auto* sTp = reinterpret_cast<float*>(sT.p);
  size_t n = g_log.size();
  expect_status("rowgroup ok", fp8_quantize_rowgroup(xp, 8, 256, 256, q.p, 256, sp, 0, nullptr), 0, n);
  CHECK(g_log.size() == n + 1 && g_log.back().kind == "rowgroup" && g_log.back().a == 8 && !g_log.back().fp32_scale,
        "rowgroup launch");
  n = g_log.size();
  expect_status("rowgroup fp32", fp8_quantize_rowgroup(xp, 8, 256, 256, q.p, 256, sp, 1, nullptr), 0, n);
  CHECK(g_log.back().fp32_scale, "rowgroup fp32 scale flag");
  n = g_log.size();
  expect_status("rowgroup mode", fp8_quantize_rowgroup(xp, 8, 256, 256, q.p, 256, sp, 2, nullptr), FP8BLK_ERR_ARG, n);
  expect_status("rowgroup null", fp8_quantize_rowgroup(nullptr, 8, 256, 256, q.p, 256, sp, 0, nullptr),
                FP8BLK_ERR_NULL, n);
  expect_status("rowgroup ragged", fp8_quantize_rowgroup(xp, 8, 200, 256, q.p, 256, sp, 0, nullptr), FP8BLK_ERR_DIM,
                n);
  expect_status("rowgroup ld", fp8_quantize_rowgroup(xp, 8, 256, 128, q.p, 256, sp, 0, nullptr), FP8BLK_ERR_ARG, n);
  expect_status("rowgroup align", fp8_quantize_rowgroup(xp + 1, 8, 256, 256, q.p, 256, sp, 0, nullptr),
                FP8BLK_ERR_ALIGN, n);
  expect_status("rowgroup huge", fp8_quantize_rowgroup(xp, int64_t(1) << 61, 128, 128, q.p, 128, sp, 0, nullptr),
                FP8BLK_ERR_ARG, n);
  expect_status("colgroup ok", fp8_quantize_colgroup(xp, 128, 256, 256, qT.p, 128, sTp, 0, nullptr), 0, n);
  n = g_log.size();
  expect_status("colgroup rows", fp8_quantize_colgroup(xp, 100, 256, 256, qT.p, 128, sTp, 0, nullptr),
                FP8BLK_ERR_DIM, n);
  expect_status("dual ok", fp8_quantize_dual(xp, 128, 256, 256, q.p, 256, sp, qT.p, 128, sTp, 0, nullptr), 0, n);
  n = g_log.size();
  expect_status("dual ld_qT", fp8_quantize_dual(xp, 128, 256, 256, q.p, 256, sp, qT.p, 64, sTp, 0, nullptr),
                FP8BLK_ERR_ARG, n);
  expect_status("block ok", fp8_quantize_block(xp, 128, 256, 256, q.p, nullptr, sp, 0, nullptr), 0, n);
  CHECK(g_log.back().kind == "block" && g_log.back().c == 0, "block launch without the transposed copy");
  n = g_log.size();
  fp8blk_block_job jobs[9];
  for (auto& j : jobs) j = fp8blk_block_job{xp, 128, 128, 128, q.p, nullptr, sp};
  expect_status("batch ok", fp8_quantize_block_batch(jobs, 8, 0, nullptr), 0, n);
  CHECK(g_log.back().kind == "block_batch" && g_log.back().a == 8, "batch launch");
  n = g_log.size();
  expect_status("batch 9", fp8_quantize_block_batch(jobs, 9, 0, nullptr), FP8BLK_ERR_ARG, n);
  jobs[3].rows = 100;
  expect_status("batch bad job", fp8_quantize_block_batch(jobs, 8, 0, nullptr), FP8BLK_ERR_DIM, n);
}

static void gemm_checks() {
  const int64_t M = 8192, N = 2048, K = 2048;
  Buf a(16), b(16), sa(16), sb(16), out(16);
  const float* sap = reinterpret_cast<const float*>(sa.p);
  const float* sbp = reinterpret_cast<const float*>(sb.p);
  size_t n = g_log.size();
  // named Fprop: the block-scaled MFMA path, contraction I = M, J = N, R = K
  expect_status("fprop", fp8_block_gemm_fprop(M, N, K, a.p, sap, b.p, sbp, out.p, FP8BLK_OUT_BF16, nullptr), 0, n);
  CHECK(g_log.size() == n + 1 && g_log.back().kind == "gemm" && g_log.back().algo == (int)fp8blk::GemmAlgo::ScaledMfma,
        "fprop launch");
  CHECK(g_log.back().g.I == M && g_log.back().g.J == N && g_log.back().g.R == K &&
            g_log.back().g.bmode == fp8blk::BScale::Block && g_log.back().g.sb_j == K / 128,
        "fprop arguments");
  // Dgrad from qw: I = M, J = K, R = N, B read transposed
  n = g_log.size();
  expect_status("dgrad_w", fp8_block_gemm_dgrad_w(M, N, K, a.p, sap, b.p, sbp, out.p, FP8BLK_OUT_FP32, nullptr), 0, n);
  CHECK(g_log.back().g.bt && g_log.back().g.I == M && g_log.back().g.J == K && g_log.back().g.R == N &&
            g_log.back().g.out_f32 && !g_log.back().g.accumulate,
        "dgrad_w arguments");
  // Wgrad needs its workspace here (tiles shared by several workgroups)
  const size_t need = fp8_block_gemm_workspace_size(FP8BLK_OP_WGRAD, M, N, K);
  CHECK(need > 0 && need != (size_t)-1, "wgrad workspace");
  Buf ws(need);
  n = g_log.size();
  expect_status("wgrad no ws", fp8_block_gemm_wgrad(M, N, K, a.p, sap, b.p, sbp, out.p, 0, nullptr, 0, nullptr),
                FP8BLK_ERR_WORKSPACE, n);
  expect_status("wgrad short ws",
                fp8_block_gemm_wgrad(M, N, K, a.p, sap, b.p, sbp, out.p, 0, ws.p, need - 1, nullptr),
                FP8BLK_ERR_WORKSPACE, n);
  expect_status("wgrad", fp8_block_gemm_wgrad(M, N, K, a.p, sap, b.p, sbp, out.p, 2, ws.p, need, nullptr), 0, n);
  CHECK(g_log.back().g.I == N && g_log.back().g.J == K && g_log.back().g.R == M &&
            g_log.back().g.bmode == fp8blk::BScale::Row && g_log.back().g.accumulate && g_log.back().g.ws != nullptr,
        "wgrad arguments");
  // the scale rule decides the algorithm
  for (int op : {FP8BLK_OP_FPROP, FP8BLK_OP_DGRAD, FP8BLK_OP_WGRAD, FP8BLK_OP_DGRAD_W}) {
    n = g_log.size();
    expect_status("fp32 scales, scaled MFMA",
                  fp8_block_gemm(op, M, N, K, a.p, sap, b.p, sbp, out.p, 0, FP8BLK_ALGO_SCALED_MFMA, FP8BLK_SCALE_FP32,
                                 ws.p, need, nullptr),
                  FP8BLK_ERR_ARG, n);
    expect_status("fp32 scales, default",
                  fp8_block_gemm(op, M, N, K, a.p, sap, b.p, sbp, out.p, 0, FP8BLK_ALGO_DEFAULT, FP8BLK_SCALE_FP32,
                                 ws.p, need, nullptr),
                  0, n);
    CHECK(g_log.back().algo == (int)fp8blk::GemmAlgo::Promote, "fp32 scales must run the promote algorithm");
    n = g_log.size();
    expect_status("pow2 scales, default",
                  fp8_block_gemm(op, M, N, K, a.p, sap, b.p, sbp, out.p, 0, FP8BLK_ALGO_DEFAULT, FP8BLK_SCALE_POW2,
                                 ws.p, need, nullptr),
                  0, n);
    CHECK(g_log.back().algo == (int)fp8blk::GemmAlgo::ScaledMfma, "power-of-two scales: the block-scaled MFMA");
    n = g_log.size();
    expect_status("bad scale mode",
                  fp8_block_gemm(op, M, N, K, a.p, sap, b.p, sbp, out.p, 0, FP8BLK_ALGO_DEFAULT, 3, ws.p, need,
                                 nullptr),
                  FP8BLK_ERR_ARG, n);
  }
  // the fused backward, and its promote pair for amax / 448 scales
  const size_t bneed = fp8_block_gemm_workspace_size(FP8BLK_OP_BACKWARD, M, N, K);
  Buf bws(bneed), dx(16), dw(16);
  n = g_log.size();
  expect_status("backward_w pow2",
                fp8_block_gemm_backward_w(M, N, K, a.p, sap, b.p, sbp, a.p, sap, b.p, sbp, dx.p, 0, dw.p, 1,
                                          FP8BLK_SCALE_POW2, bws.p, bneed, nullptr),
                0, n);
  CHECK(g_log.size() == n + 1 && g_log.back().kind == "gemm_mx_bwd" && g_log.back().g.bt &&
            g_log.back().g2.ws != nullptr,
        "backward_w: one fused launch");
  n = g_log.size();
  expect_status("backward fp32",
                fp8_block_gemm_backward(M, N, K, a.p, sap, b.p, sbp, a.p, sap, b.p, sbp, dx.p, 0, dw.p, 1,
                                        FP8BLK_SCALE_FP32, bws.p, bneed, nullptr),
                0, n);
  CHECK(g_log.size() == n + 2 && g_log[n].algo == (int)fp8blk::GemmAlgo::Promote &&
            g_log[n + 1].algo == (int)fp8blk::GemmAlgo::Promote && g_log[n + 1].g.bmode == fp8blk::BScale::Row,
        "backward with fp32 scales: two promote launches, Dgrad then Wgrad");
  n = g_log.size();
  expect_status("backward alias",
                fp8_block_gemm_backward(M, N, K, a.p, sap, b.p, sbp, a.p, sap, b.p, sbp, dx.p, 0, dx.p, 1,
                                        FP8BLK_SCALE_POW2, bws.p, bneed, nullptr),
                FP8BLK_ERR_ARG, n);
  expect_status("backward mode",
                fp8_block_gemm_backward(M, N, K, a.p, sap, b.p, sbp, a.p, sap, b.p, sbp, dx.p, 0, dw.p, 1, 5, bws.p,
                                        bneed, nullptr),
                FP8BLK_ERR_ARG, n);
  expect_status("backward short ws",
                fp8_block_gemm_backward(M, N, K, a.p, sap, b.p, sbp, a.p, sap, b.p, sbp, dx.p, 0, dw.p, 1,
                                        FP8BLK_SCALE_POW2, bws.p, bneed - 16, nullptr),
                FP8BLK_ERR_WORKSPACE, n);
  // the no-allocation form: the same launches, the static scratch as workspace
  n = g_log.size();
  expect_status("noalloc pow2",
                fp8_block_gemm_backward_w_noalloc(M, N, K, a.p, sap, b.p, sbp, a.p, sap, b.p, sbp, dx.p, 0, dw.p, 1,
                                                  FP8BLK_SCALE_POW2, nullptr),
                0, n);
  CHECK(g_log.size() == n + 1 && g_log.back().kind == "gemm_mx_bwd" && g_log.back().g.bt &&
            (void*)g_log.back().g2.ws == (void*)fp8blk::g_fake_scratch,
        "noalloc: the fused launch on the static scratch");
  n = g_log.size();
  expect_status("noalloc too big",
                fp8_block_gemm_backward_w_noalloc(1536, 1536, 2560, a.p, sap, b.p, sbp, a.p, sap, b.p, sbp, dx.p, 0,
                                                  dw.p, 1, FP8BLK_SCALE_POW2, nullptr),
                FP8BLK_ERR_SCRATCH, n);
  expect_status("noalloc fp32",
                fp8_block_gemm_backward_w_noalloc(M, N, K, a.p, sap, b.p, sbp, a.p, sap, b.p, sbp, dx.p, 0, dw.p, 1,
                                                  FP8BLK_SCALE_FP32, nullptr),
                0, n);
  CHECK(g_log.size() == n + 2 && g_log[n].algo == (int)fp8blk::GemmAlgo::Promote && g_log[n].g.bt,
        "noalloc fp32: the promote pair");
  n = g_log.size();
  expect_status("noalloc alias",
                fp8_block_gemm_backward_w_noalloc(M, N, K, a.p, sap, b.p, sbp, a.p, sap, b.p, sbp, dw.p, 0, dw.p, 1,
                                                  FP8BLK_SCALE_POW2, nullptr),
                FP8BLK_ERR_ARG, n);
  CHECK(fp8_block_gemm_workspace_size(9, M, N, K) == (size_t)-1, "bad op");
  CHECK(fp8_block_gemm_workspace_size(FP8BLK_OP_FPROP, 100, N, K) == (size_t)-1, "bad shape");
  for (int st = 1; st >= -9; --st) CHECK(fp8_status_string(st) != nullptr, "status string");
  CHECK(std::strstr(fp8_status_string(FP8BLK_ERR_SCRATCH), "scratch") != nullptr, "scratch status string");
}

// ---- slot tables: a host mirror of the kernels' walk (gemm_mx.hip).

// Slot of range r's first or last partial segment, as the kernels compute it.
static int64_t slot_of(const uint16_t* t, int64_t r, bool first) {
  return (int64_t)(t[r] >> 1) + (first ? 0 : (int64_t)(t[r] & 1));
}

// Walk every range [rs[r], rs[r+1]) of W units over problems [0, w0) (tiles
// of u0 units) and [w0, W) (u1) as the kernels do; check that every unit of
// every tile is reduced exactly once, mapping a dealt problem's segments to
// tiles as the backward kernel does (deal, rp0, rpn: BwdGeom's; all zero for
// the Wgrad plans), and that dealt tiles are never shared.  Record for every
// partial segment (problem, tile, first unit) the slot its range writes;
// then enumerate each shared tile's pieces as the fix-up does and check that
// piece k is the slot that wrote units [piece start ..).
static void check_slots(const char* what, const uint16_t* table, int64_t slots, int64_t G, int64_t W, int64_t w0,
                        int64_t u0, int64_t u1, const uint32_t* rs, const int64_t* deal = nullptr,
                        const int64_t* rp0 = nullptr, const int64_t* rpn = nullptr) {
  CHECK(rs[0] == 0 && (int64_t)rs[G] == W, "%s: ranges cover [%u, %u), not [0, %lld)", what, rs[0], rs[G],
        (long long)W);
  for (int64_t r = 0; r < G; ++r)
    CHECK(rs[r] < rs[r + 1], "%s: range %lld is empty or reversed", what, (long long)r);
  std::set<int64_t> used;
  // (unit of the piece's start) -> slot
  std::vector<int64_t> slot_at(W, -1);
  // units reduced per tile, problem 0's tiles then problem 1's
  const int64_t t0 = w0 / u0, t1 = u1 > 0 ? (W - w0) / u1 : 0;
  std::vector<int64_t> cov(t0 + t1, 0);
  for (int64_t r = 0; r < G; ++r) {
    const int64_t ubeg = rs[r], uend = rs[r + 1];
    for (int64_t u = ubeg; u < uend;) {
      const bool p1 = u >= w0;
      const int64_t base = p1 ? w0 : 0, U = p1 ? u1 : u0;
      const int64_t ts = (u - base) / U, lo = u - base - ts * U;
      const int64_t tend = base + (ts + 1) * U;
      const int64_t hi = (uend < tend ? uend : tend) - base - ts * U;
      const int q = p1 ? 1 : 0;
      const bool dealt = deal != nullptr && deal[q] != 0;
      const int64_t tt = dealt ? ((u - ubeg) / U) * rpn[q] + (r - rp0[q]) : ts;
      CHECK(tt >= 0 && tt < (p1 ? t1 : t0), "%s: range %lld maps a segment to tile %lld of %lld", what,
            (long long)r, (long long)tt, (long long)(p1 ? t1 : t0));
      if (tt >= 0 && tt < (p1 ? t1 : t0)) cov[(p1 ? t0 : 0) + tt] += hi - lo;
      if (!(lo == 0 && hi == U)) {
        CHECK(!dealt, "%s: range %lld holds part of a dealt tile", what, (long long)r);
        const int64_t s = slot_of(table, r, u == ubeg);
        CHECK(s >= 0 && s < slots, "%s: range %lld writes slot %lld outside [0, %lld)", what, (long long)r,
              (long long)s, (long long)slots);
        CHECK(used.insert(s).second, "%s: slot %lld written twice", what, (long long)s);
        slot_at[u] = s;
      }
      u = base + ts * U + hi;
    }
  }
  for (int64_t t = 0; t < t0 + t1; ++t)
    CHECK(cov[t] == (t < t0 ? u0 : u1), "%s: tile %lld reduced over %lld units", what, (long long)t,
          (long long)cov[t]);
  CHECK((int64_t)used.size() == slots, "%s: %zu slots written, plan says %lld", what, used.size(), (long long)slots);
  // the fix-up: tile starting at unit `first` with U units
  auto fixup = [&](int64_t first, int64_t U) {
    const int64_t f = fp8blk::h_range_of(rs, G, first);
    const int64_t pieces = fp8blk::h_range_of(rs, G, first + U - 1) - f + 1;
    if (pieces == 1) return;
    for (int64_t pc = 0; pc < pieces; ++pc) {
      const int64_t s = pc == 0 ? slot_of(table, f, !((int64_t)rs[f] < first)) : slot_of(table, f + pc, true);
      const int64_t start = pc == 0 ? first : (int64_t)rs[f + pc];
      CHECK(start < W && slot_at[start] == s, "%s: fix-up of the tile at unit %lld reads slot %lld for piece %lld",
            what, (long long)first, (long long)s, (long long)pc);
    }
  };
  for (int64_t u = 0; u < w0; u += u0) fixup(u, u0);
  for (int64_t u = w0; u < W; u += u1) fixup(u, u1);
}

// The Wgrad kernels' even cut: range w of Gs over W units starts at w W / Gs.
static std::vector<uint32_t> even_ranges(int64_t W, int64_t G) {
  std::vector<uint32_t> rs(G + 1);
  for (int64_t w = 0; w <= G; ++w) rs[w] = (uint32_t)fp8blk::h_start(w, W, G);
  return rs;
}

static void plan_checks() {
  // (M, N, K) of the decoder layer's linears, the smaller test shapes and a
  // few whose ranges split tiles unevenly
  const int64_t shapes[][3] = {{8192, 4096, 2048}, {8192, 2048, 2048}, {8192, 12288, 2048}, {8192, 2048, 6144},
                               {1024, 1536, 1024}, {2048, 1536, 1152}, {512, 1024, 640},   {1024, 512, 384},
                               {9216, 1152, 768},  {2048, 256, 256},   {1024, 4096, 6144}, {512, 5120, 7680},
                               {2048, 4352, 4096}, {4608, 2560, 1408}, {2560, 6656, 896},  {512, 512, 128},
                               {384, 640, 512},    {640, 384, 1024},   {1024, 2560, 3840}, {128, 384, 256}};
  for (const auto& sh : shapes) {
    const int64_t M = sh[0], N = sh[1], K = sh[2];
    char what[96];
    if ((M / 128) % 4 == 0 && (N / 128) % 4 == 0) {
      const fp8blk::BwdPlan p = fp8blk::bwd_plan(M, N, K);
      std::snprintf(what, sizeof what, "backward %lldx%lldx%lld", (long long)M, (long long)N, (long long)K);
      const fp8blk::BwdGeom& g = p.geom;
      check_slots(what, g.slot, p.slots, p.grid, g.units, g.w0, g.u0, g.u1, g.rstart, g.deal, g.rp0, g.rpn);
      CHECK(g.t0 == g.tm0 * g.tn0 && g.w0 == g.t0 * g.u0 && g.units == g.w0 + g.tm1 * g.tn1 * g.u1,
            "%s: geometry", what);
      // the shared-tile list: exactly the tiles spanning more than one range, ascending
      std::vector<uint32_t> want;
      for (int64_t t = 0; t < g.t0 + g.tm1 * g.tn1; ++t) {
        const bool p1 = t >= g.t0;
        const int64_t U = p1 ? g.u1 : g.u0, first = p1 ? g.w0 + (t - g.t0) * U : t * U;
        if (fp8blk::h_range_of(g.rstart, p.grid, first) != fp8blk::h_range_of(g.rstart, p.grid, first + U - 1))
          want.push_back((uint32_t)t);
      }
      CHECK(g.nshared == (int64_t)want.size() && std::equal(want.begin(), want.end(), g.shared),
            "%s: %lld shared tiles listed, %zu span several ranges", what, (long long)g.nshared, want.size());
      CHECK((p.slots == 0) == (g.nshared == 0), "%s: slots without shared tiles or the reverse", what);
      CHECK(p.bytes == (size_t)p.slots * 256 * 256 * 4, "%s: bytes", what);
    }
    {  // the general kernel's Wgrad: 256 x 128 tiles, units of 4 or 1 blocks
      const fp8blk::SkPlan p = fp8blk::general_sk_plan(N, K, M);
      std::snprintf(what, sizeof what, "general wgrad %lldx%lldx%lld", (long long)M, (long long)N, (long long)K);
      const int64_t U = M / (128 * p.geom.ublocks);
      CHECK(p.geom.ublocks == ((M / 128) % 4 == 0 ? 4 : 1), "%s: unit size", what);
      if (p.geom.units > 0)
        check_slots(what, p.geom.slot, p.slots, p.geom.sk_grid, p.geom.units, p.geom.units, U, U,
                    even_ranges(p.geom.units, p.geom.sk_grid).data());
      else
        CHECK(p.slots == 0, "%s: no stream-K units, no slots", what);
      CHECK(p.bytes == (size_t)p.slots * 256 * 128 * 4, "%s: bytes", what);
      CHECK(p.slots <= 2 * fp8blk::kSkGrid, "%s: at most two partial segments per range", what);
    }
    if ((M / 128) % 4 == 0) {
      const fp8blk::SkPlan p = fp8blk::sk_plan(N, K, M);  // Wgrad: I = N, J = K, R = M
      std::snprintf(what, sizeof what, "wgrad %lldx%lldx%lld", (long long)M, (long long)N, (long long)K);
      if (p.geom.units > 0)
        check_slots(what, p.geom.slot, p.slots, p.geom.sk_grid, p.geom.units, p.geom.units, M / 512, M / 512,
                    even_ranges(p.geom.units, p.geom.sk_grid).data());
      else
        CHECK(p.slots == 0, "%s: no stream-K units, no slots", what);
    }
  }
  // the decoder layer's backward launches: at most 128 partial tiles each
  for (const auto& sh : shapes) {
    if (sh[0] != 8192) continue;
    const fp8blk::BwdPlan p = fp8blk::bwd_plan(sh[0], sh[1], sh[2]);
    CHECK(p.slots <= 128, "layer backward %lldx%lld: %lld slots", (long long)sh[1], (long long)sh[2],
          (long long)p.slots);
  }
}

int main() {
  quantizer_checks();
  gemm_checks();
  plan_checks();
  if (g_fail == 0) std::printf("ok\n");
  return g_fail == 0 ? 0 : 1;
}
