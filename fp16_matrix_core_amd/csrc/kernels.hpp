// kernels.hpp -- internal interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp16mc {

// Element types; the values equal fp16mc_dtype of the C header.
enum class Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// One batched product: problem b reads A + b*sA, B + b*sB, writes Out + b*sO
// (strides in elements).  A and B hold ab_type (F16 or BF16); Out holds
// out_type (F32 or ab_type); with `accumulate` Out's previous values are added.
// a_mn / b_mn: the operand is stored with K indexing its rows (A[k*lda + i],
// B[k*ldb + j]) instead of K-contiguous rows (A[i*lda + k], B[j*ldb + k]).
struct GemmProblem {
  const void* A;
  const void* B;
  void* Out;
  int64_t M, N, K;
  int64_t lda, ldb, ldo;
  int64_t batch;
  int64_t sA, sB, sO;
  Dtype ab_type;
  Dtype out_type;
  bool accumulate;
  bool a_mn;
  bool b_mn;
};

// Kernel configurations, one per shape class.
enum class GemmPlan : int {
  kNone = 0,      // empty problem, nothing to launch
  kWave32 = 1,    // one wavefront per 32x32 output tile (tiny problems)
  kWg128x64 = 2,        // 4 wavefronts per 128x64 tile (small and mid-size)
  kWg256 = 3,           // 4 wavefronts per 256x256 tile (large problems)
  kTall = 4,            // N <= 32: 2 wavefronts per 64x32 tile, A streamed
  kWg128x64Stream = 5,  // batches of one-tile problems: 128x64 tiles, both operands streamed
  kWg256x128 = 6,       // 4 wavefronts per 256x128 tile
  kWg128x128 = 7,       // 4 wavefronts per 128x128 tile, two workgroups per CU
  kWide = 8,            // M <= 32: 2 wavefronts per 32x64 tile, B streamed
  kWg64 = 9,            // 4 wavefronts per 64x64 tile (at most one tile per CU)
};

GemmPlan choose_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t batch, bool a_mn, bool b_mn);
// The plan's kernel name for one storage order of the operands (a_mn / b_mn:
// A / B stored with M / N contiguous).
const char* gemm_plan_name(GemmPlan plan, bool a_mn, bool b_mn);
// Number of workgroups the plan launches (host-side; used to validate the grid).
int64_t gemm_plan_grid(GemmPlan plan, int64_t M, int64_t N, int64_t batch);
hipError_t launch_gemm(GemmPlan plan, const GemmProblem& p, hipStream_t stream);
// One storage order each (gemm_nt.hip, gemm_nn.hip, gemm_tt.hip, gemm_tn.hip).
hipError_t launch_gemm_nt(GemmPlan plan, const GemmProblem& p, hipStream_t stream);
hipError_t launch_gemm_nn(GemmPlan plan, const GemmProblem& p, hipStream_t stream);
hipError_t launch_gemm_tt(GemmPlan plan, const GemmProblem& p, hipStream_t stream);
hipError_t launch_gemm_tn(GemmPlan plan, const GemmProblem& p, hipStream_t stream);
// True when every operand tile of the plan spans fewer than 2^32 bytes and a
// tile's rows of Out (out_bytes per element) fewer than 2^31 (the kernels
// address a tile through a buffer descriptor with 32-bit offsets).
bool gemm_plan_fits_offsets(GemmPlan plan, int64_t K, int64_t lda, int64_t ldb, int64_t ldo, int64_t out_bytes,
                            bool a_mn, bool b_mn);

// Fragment copy; `groups` = num_tiles / num.
hipError_t launch_frag_copy(const void* src, void* dst, int64_t groups, int num, bool col_major,
                            int direction, hipStream_t stream);

}  // namespace fp16mc
