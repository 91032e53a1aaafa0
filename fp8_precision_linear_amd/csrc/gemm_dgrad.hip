// FP8 product kernels, data gradient: W8 read with the contraction as its slow index.
// One translation unit per operand layout so the instantiations compile in parallel.
#include "gemm_group.h"

namespace fp8lin {

hipError_t launch_gemm_dgrad(const GemmProblem& p, hipStream_t stream) {
  return gemm_detail::launch_layout<true, false>(p, stream);
}

hipError_t launch_gemm_dgrad_ws(const GemmProblem& p, float* ws, int64_t max_bytes, hipStream_t stream) {
  return gemm_detail::launch_layout_ws<true, false>(p, ws, max_bytes, stream);
}

hipError_t launch_gemm_dgrad_group(const GemmProblem* ps, const GroupSlot* plan, const int* idx, int n,
                                   uint8_t* ws, hipStream_t stream) {
  return gemm_detail::launch_group_layout<true, false>(ps, plan, idx, n, ws, stream);
}

}  // namespace fp8lin
