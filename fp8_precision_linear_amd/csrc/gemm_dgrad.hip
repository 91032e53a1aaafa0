// FP8 product kernels, data gradient: W8 read with the contraction as its slow index.
// One translation unit per operand layout so the instantiations compile in parallel.
#include "gemm_pipe.h"

namespace fp8lin {

hipError_t launch_gemm_dgrad(const GemmProblem& p, hipStream_t stream) {
  return gemm_detail::launch_layout<true, false>(p, stream);
}

}  // namespace fp8lin
