// gemm_nn.hip -- kernels for operands A (M, K) K-contiguous, B stored (K, N) with N contiguous: Out = A @ B
// (gemm_kernels.hpp holds the templates).

#include "gemm_kernels.hpp"

namespace fp16mc {

hipError_t launch_gemm_nn(GemmPlan plan, const GemmProblem& p, hipStream_t stream) {
  return launch_layout<false, true>(plan, p, stream);
}

}  // namespace fp16mc
