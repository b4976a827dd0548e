// gemm_nt.hip -- kernels for operands A (M, K) and B (N, K), both K-contiguous: Out = A @ B.T
// (gemm_kernels.hpp holds the templates).

#include "gemm_kernels.hpp"

namespace fp16mc {

hipError_t launch_gemm_nt(GemmPlan plan, const GemmProblem& p, hipStream_t stream) {
  return launch_layout<false, false>(plan, p, stream);
}

}  // namespace fp16mc
