// gemm_tn.hip -- kernels for operands A stored (K, M) and B stored (K, N), both M/N-contiguous: Out = A.T @ B
// (gemm_kernels.hpp holds the templates).

#include "gemm_kernels.hpp"

namespace fp16mc {

hipError_t launch_gemm_tn(GemmPlan plan, const GemmProblem& p, hipStream_t stream) {
  return launch_layout<true, true>(plan, p, stream);
}

}  // namespace fp16mc
