// FP8 product kernels, forward: both operands contraction-contiguous.
// One translation unit per operand layout so the instantiations compile in parallel.
#include "gemm_pipe.h"

namespace fp8lin {

hipError_t launch_gemm_fwd(const GemmProblem& p, hipStream_t stream) {
  return gemm_detail::launch_layout<true, true>(p, stream);
}

}  // namespace fp8lin
