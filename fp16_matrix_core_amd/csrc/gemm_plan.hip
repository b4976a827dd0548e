// gemm_plan.hip -- host side of the product: which kernel configuration a
// problem gets, its grid, its addressing limits, and the dispatch to the
// source file that instantiates the operands' storage order.

#include <cmath>

#include "gemm_kernels.hpp"

namespace fp16mc {

namespace {

// Ranking model of the tile configurations (fp16 -> fp32, NT): a rate at
// full occupancy, the K at which the per-tile prologue and epilogue cost as
// much as the K loop, and how many workgroups fit on a CU.  The rate and k0
// pairs are fitted so that the model picks the fastest configuration of a
// forced-plan sweep on MI355X (17 shapes from 1024^3 to 12288^2 x 1024; it
// misses one, 8192^2 x 1024, by 4%); they rank configurations, they are not
// the configurations' measured peak rates.
struct TileModel {
  GemmPlan plan;
  int bm, bn;
  double tflops;     // rate at full occupancy, K >> k0
  double k0;         // per-tile overhead expressed in K
  int per_cu;        // workgroups per CU (LDS)
};
constexpr TileModel kModels[] = {
    {GemmPlan::kWg256, 256, 256, 1150.0, 300.0, 1},
    {GemmPlan::kWg256x128, 256, 128, 1075.0, 275.0, 1},
    {GemmPlan::kWg128x128, 128, 128, 1060.0, 200.0, 2},
    {GemmPlan::kWg128x64, 128, 64, 870.0, 220.0, 2},
};

// Predicted useful rate: the full-occupancy rate, discounted for the
// per-tile overhead, for idle CUs in the last wave of tiles, and for the part
// of the edge tiles that lies outside M x N.  A partly filled chip runs at a
// higher clock (the product is power-limited), hence the 0.75 power on the
// fill fraction (fitted to the measured rates).
double predicted_rate(const TileModel& m, int64_t M, int64_t N, int64_t K, int64_t batch) {
  const int64_t tm = (M + m.bm - 1) / m.bm, tn = (N + m.bn - 1) / m.bn;
  const double tiles = double(tm) * double(tn) * double(batch);
  const double slots = 256.0 * m.per_cu;
  const double waves = std::ceil(tiles / slots);
  const double fill = tiles / (waves * slots);
  const double useful = (double(M) / double(tm * m.bm)) * (double(N) / double(tn * m.bn));
  return m.tflops * (double(K) / (double(K) + m.k0)) * std::pow(fill, 0.75) * useful;
}

}  // namespace

GemmPlan choose_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t batch, bool /*a_mn*/, bool /*b_mn*/) {
  if (M <= 0 || N <= 0 || batch <= 0) return GemmPlan::kNone;
  if (M <= 32 && N <= 32) return GemmPlan::kWave32;
  // N <= 32: one column of tall tiles streams A past a shared B; M <= 32: the mirror
  if (N <= 32) return GemmPlan::kTall;
  if (M <= 32) return GemmPlan::kWide;
  // a batch of one-tile problems: nothing is read twice
  if (batch > 1 && M <= 128 && N <= 64) return GemmPlan::kWg128x64Stream;
  // At most 256 tiles of 64x64 (K >= 512): the larger tiles would occupy a
  // fraction of the CUs; 64x64 tiles give each CU at most one (1024^2 x 4096
  // 22 -> 15 us, 768^2 x 2048 9.8 -> 7.0 us, 512^2 x 16384 69 -> 42 us).
  if (K >= 512 && double((M + 63) / 64) * double((N + 63) / 64) * double(batch) <= 256.0) return GemmPlan::kWg64;
  GemmPlan best = GemmPlan::kWg128x64;
  double best_rate = -1.0;
  for (const TileModel& m : kModels) {
    const double r = predicted_rate(m, M, N, K > 0 ? K : 1, batch);
    if (r > best_rate) {
      best_rate = r;
      best = m.plan;
    }
  }
  return best;
}

const char* gemm_plan_name(GemmPlan plan, bool a_mn, bool b_mn) {
  const bool mn = a_mn || b_mn;   // large tiles: 16x16x32 for K-contiguous operands, else 32x32x16
  switch (plan) {
    case GemmPlan::kWave32: return "wave32x32_mfma32x32x16";
    case GemmPlan::kWg128x64: return mn ? "wg128x64_w4_mfma32x32x16" : "wg128x64_w4_mfma16x16x32";
    case GemmPlan::kWg256: return "wg256x256_w4_mfma16x16x32";
    case GemmPlan::kTall: return "tall64x32_w2_mfma32x32x16";
    case GemmPlan::kWg128x64Stream: return "wg128x64s_w4_mfma32x32x16";
    case GemmPlan::kWg256x128: return "wg256x128_w4_mfma16x16x32";
    case GemmPlan::kWg128x128: return "wg128x128_w4_mfma16x16x32";
    case GemmPlan::kWide: return "wide32x64_w2_mfma32x32x16";
    case GemmPlan::kWg64: return mn ? "wg64x64_w4_mfma32x32x16" : "wg64x64_w4_mfma16x16x32";
    default: return nullptr;
  }
}

// Workgroups of the launch, saturated at INT64_MAX instead of wrapping (the
// caller rejects anything above its grid limit).
template <class C>
int64_t grid_of(int64_t M, int64_t N, int64_t batch) {
  const int64_t tm = M / C::BM + (M % C::BM != 0);
  const int64_t tn = N / C::BN + (N % C::BN != 0);
  int64_t t = 0;
  if (__builtin_mul_overflow(tm, tn, &t) || __builtin_mul_overflow(t, batch, &t)) return INT64_MAX;
  return t;
}

int64_t gemm_plan_grid(GemmPlan plan, int64_t M, int64_t N, int64_t batch) {
  switch (plan) {
    case GemmPlan::kWave32: return grid_of<CfgWave32>(M, N, batch);
    case GemmPlan::kWg128x64: return grid_of<CfgWg128x64>(M, N, batch);
    case GemmPlan::kWg256: return grid_of<CfgWg256>(M, N, batch);
    case GemmPlan::kTall: return grid_of<CfgTall>(M, N, batch);
    case GemmPlan::kWg128x64Stream: return grid_of<CfgWg128x64Stream>(M, N, batch);
    case GemmPlan::kWg256x128: return grid_of<CfgWg256x128>(M, N, batch);
    case GemmPlan::kWg128x128: return grid_of<CfgWg128x128>(M, N, batch);
    case GemmPlan::kWide: return grid_of<CfgWide>(M, N, batch);
    case GemmPlan::kWg64: return grid_of<CfgWg64>(M, N, batch);
    default: return 0;
  }
}

// The kernels address an operand through buffer descriptors with 32-bit byte
// offsets: a K-contiguous tile spans W - 1 rows plus K values; an
// MN-contiguous one is re-based for every slice and spans BK rows.
template <class C>
bool fits_offsets(int64_t K, int64_t lda, int64_t ldb, int64_t ldo, int64_t out_bytes, bool a_mn, bool b_mn) {
  const int64_t limit = int64_t(1) << 32;
  // Larger values fail below anyway; bounding them first keeps the products in range.
  if (K >= limit || lda >= limit || ldb >= limit || ldo >= (int64_t(1) << 31)) return false;
  const int64_t a = a_mn ? 2 * C::BK * lda : 2 * ((C::BM - 1) * lda + K);
  const int64_t b = b_mn ? 2 * C::BK * ldb : 2 * ((C::BN - 1) * ldb + K);
  // Out is addressed from each tile's origin with signed 32-bit row offsets
  const int64_t o = int64_t(C::BM) * ldo * out_bytes;
  return a < limit && b < limit && o < (int64_t(1) << 31);
}

bool gemm_plan_fits_offsets(GemmPlan plan, int64_t K, int64_t lda, int64_t ldb, int64_t ldo, int64_t out_bytes,
                            bool a_mn, bool b_mn) {
  switch (plan) {
    case GemmPlan::kWave32: return fits_offsets<CfgWave32>(K, lda, ldb, ldo, out_bytes, a_mn, b_mn);
    case GemmPlan::kWg128x64: return fits_offsets<CfgWg128x64>(K, lda, ldb, ldo, out_bytes, a_mn, b_mn);
    case GemmPlan::kWg256: return fits_offsets<CfgWg256>(K, lda, ldb, ldo, out_bytes, a_mn, b_mn);
    case GemmPlan::kTall: return fits_offsets<CfgTall>(K, lda, ldb, ldo, out_bytes, a_mn, b_mn);
    case GemmPlan::kWg128x64Stream: return fits_offsets<CfgWg128x64Stream>(K, lda, ldb, ldo, out_bytes, a_mn, b_mn);
    case GemmPlan::kWg256x128: return fits_offsets<CfgWg256x128>(K, lda, ldb, ldo, out_bytes, a_mn, b_mn);
    case GemmPlan::kWg128x128: return fits_offsets<CfgWg128x128>(K, lda, ldb, ldo, out_bytes, a_mn, b_mn);
    case GemmPlan::kWide: return fits_offsets<CfgWide>(K, lda, ldb, ldo, out_bytes, a_mn, b_mn);
    case GemmPlan::kWg64: return fits_offsets<CfgWg64>(K, lda, ldb, ldo, out_bytes, a_mn, b_mn);
    default: return true;
  }
}

hipError_t launch_gemm(GemmPlan plan, const GemmProblem& p, hipStream_t stream) {
  if (plan == GemmPlan::kNone) return hipSuccess;
  if (!p.a_mn && !p.b_mn) return launch_gemm_nt(plan, p, stream);
  if (!p.a_mn && p.b_mn) return launch_gemm_nn(plan, p, stream);
  if (p.a_mn && !p.b_mn) return launch_gemm_tt(plan, p, stream);
  return launch_gemm_tn(plan, p, stream);
}

}  // namespace fp16mc
