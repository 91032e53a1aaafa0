// FP8 product kernels, forward: both operands contraction-contiguous.
// One translation unit per operand layout so the instantiations compile in parallel.
#include "gemm_split.h"

namespace fp8lin {

hipError_t launch_gemm_fwd(const GemmProblem& p, hipStream_t stream) {
  return gemm_detail::launch_layout<true, true>(p, stream);
}

hipError_t launch_gemm_fwd_ws(const GemmProblem& p, float* ws, hipStream_t stream) {
  return gemm_detail::launch_layout_ws<true, true>(p, ws, stream);
}

int64_t gemm_split_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  return gemm_detail::split_workspace_bytes(m, n, k);
}

}  // namespace fp8lin
