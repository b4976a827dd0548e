// gemm_tt.hip -- kernels for operands A stored (K, M) with M contiguous, B (N, K) K-contiguous: Out = A.T @ B.T
// (gemm_kernels.hpp holds the templates).

#include "gemm_kernels.hpp"

namespace fp16mc {

hipError_t launch_gemm_tt(GemmPlan plan, const GemmProblem& p, hipStream_t stream) {
  return launch_layout<true, false>(plan, p, stream);
}

}  // namespace fp16mc
