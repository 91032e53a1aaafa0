// FP8 product kernels, data gradient: W8 read with the contraction as its slow index.
// One translation unit per operand layout so the instantiations compile in parallel.
#include "gemm_split.h"

namespace fp8lin {

hipError_t launch_gemm_dgrad(const GemmProblem& p, hipStream_t stream) {
  return gemm_detail::launch_layout<true, false>(p, stream);
}

hipError_t launch_gemm_dgrad_ws(const GemmProblem& p, float* ws, hipStream_t stream) {
  return gemm_detail::launch_layout_ws<true, false>(p, ws, stream);
}

}  // namespace fp8lin
