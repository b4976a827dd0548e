// gemm_plan.hip -- host side of the product: which kernel configuration a
// problem gets, its grid, its addressing limits, and the dispatch to the
// source file that instantiates the operands' storage order.

#include "gemm_kernels.hpp"

namespace fp16mc {

GemmPlan choose_gemm_plan(int64_t M, int64_t N, int64_t /*K*/, int64_t batch, bool /*a_mn*/, bool /*b_mn*/) {
  if (M <= 0 || N <= 0 || batch <= 0) return GemmPlan::kNone;
  if (M <= 32 && N <= 32) return GemmPlan::kWave32;
  // N <= 32: one column of tall tiles streams A past a shared B
  if (N <= 32) return GemmPlan::kTall;
  // 256x256 tiles only where they are mostly full and there are enough of
  // them to occupy at least half of the 256 CUs.
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256) * batch;
  if (M >= 256 && N >= 256 && big_tiles >= 128) return GemmPlan::kWg256;
  // a batch of one-tile problems: nothing is read twice
  if (batch > 1 && M <= 128 && N <= 64) return GemmPlan::kWg128x64Stream;
  return GemmPlan::kWg128x64;
}

const char* gemm_plan_name(GemmPlan plan) {
  switch (plan) {
    case GemmPlan::kWave32: return "wave32x32_mfma32x32x16";
    case GemmPlan::kWg128x64: return "wg128x64_w4_mfma32x32x16";
    case GemmPlan::kWg256: return "wg256x256_w4_mfma32x32x16";
    case GemmPlan::kTall: return "tall64x32_w2_mfma32x32x16";
    case GemmPlan::kWg128x64Stream: return "wg128x64s_w4_mfma32x32x16";
    default: return nullptr;
  }
}

int64_t gemm_plan_grid(GemmPlan plan, int64_t M, int64_t N, int64_t batch) {
  int64_t tm, tn;
  switch (plan) {
    case GemmPlan::kWave32: return tiles_of<CfgWave32>(M, N, batch, &tm, &tn);
    case GemmPlan::kWg128x64: return tiles_of<CfgWg128x64>(M, N, batch, &tm, &tn);
    case GemmPlan::kWg256: return tiles_of<CfgWg256>(M, N, batch, &tm, &tn);
    case GemmPlan::kTall: return tiles_of<CfgTall>(M, N, batch, &tm, &tn);
    case GemmPlan::kWg128x64Stream: return tiles_of<CfgWg128x64Stream>(M, N, batch, &tm, &tn);
    default: return 0;
  }
}

// The kernels address an operand through buffer descriptors with 32-bit byte
// offsets: a K-contiguous tile spans W - 1 rows plus K values; an
// MN-contiguous one is re-based for every slice and spans BK rows.
template <class C>
bool fits_offsets(int64_t K, int64_t lda, int64_t ldb, bool a_mn, bool b_mn) {
  const int64_t limit = int64_t(1) << 32;
  const int64_t a = a_mn ? 2 * C::BK * lda : 2 * ((C::BM - 1) * lda + K);
  const int64_t b = b_mn ? 2 * C::BK * ldb : 2 * ((C::BN - 1) * ldb + K);
  return a < limit && b < limit;
}

bool gemm_plan_fits_offsets(GemmPlan plan, int64_t K, int64_t lda, int64_t ldb, bool a_mn, bool b_mn) {
  switch (plan) {
    case GemmPlan::kWave32: return fits_offsets<CfgWave32>(K, lda, ldb, a_mn, b_mn);
    case GemmPlan::kWg128x64: return fits_offsets<CfgWg128x64>(K, lda, ldb, a_mn, b_mn);
    case GemmPlan::kWg256: return fits_offsets<CfgWg256>(K, lda, ldb, a_mn, b_mn);
    case GemmPlan::kTall: return fits_offsets<CfgTall>(K, lda, ldb, a_mn, b_mn);
    case GemmPlan::kWg128x64Stream: return fits_offsets<CfgWg128x64Stream>(K, lda, ldb, a_mn, b_mn);
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
