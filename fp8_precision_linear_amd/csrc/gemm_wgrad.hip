// FP8 product kernels, weight gradient: both operands read with the contraction as their slow index.
// One translation unit per operand layout so the instantiations compile in parallel.
#include "gemm_split.h"

namespace fp8lin {

hipError_t launch_gemm_wgrad(const GemmProblem& p, hipStream_t stream) {
  return gemm_detail::launch_layout<false, false>(p, stream);
}

hipError_t launch_gemm_wgrad_ws(const GemmProblem& p, float* ws, hipStream_t stream) {
  return gemm_detail::launch_layout_ws<false, false>(p, ws, stream);
}

}  // namespace fp8lin
