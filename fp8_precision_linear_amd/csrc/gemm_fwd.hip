// FP8 product kernels, forward: both operands contraction-contiguous.
// One translation unit per operand layout so the instantiations compile in parallel.
#include <algorithm>

#include "gemm_group.h"

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

// Which products run grouped and how they are split: each grouped launch
// holds one layout and format pair (a bucket); within a bucket every
// product's contraction is cut into slices of about the bucket's shortest
// contraction (at least kGroupMinSliceStages stages, at most 16 slices), so
// its blocks do similar work.
int64_t gemm_group_plan(const GemmProblem* ps, int count, GroupSlot* plan) {
  using namespace gemm_detail;
  auto eligible = [](const GemmProblem& p) {
    if (p.m <= 0 || p.n <= 0 || p.ldc != p.n) return false;
    const int64_t tiles = (int64_t)((p.m + 127) / 128) * ((p.n + 127) / 128);
    if (tiles > kGroupMaxTiles) return false;
    if (p.a_kmajor && p.b_kmajor) return pipe_ok<true, true>(p);
    if (p.a_kmajor && !p.b_kmajor) return pipe_ok<true, false>(p);
    if (!p.a_kmajor && !p.b_kmajor) return pipe_ok<false, false>(p);
    return false;
  };
  auto bucket = [](const GemmProblem& p) {
    return (p.a_kmajor ? 1 : 0) + (p.b_kmajor ? 2 : 0) + 4 * (p.fmt_a == FP8_E5M2 ? 1 : 0) +
           8 * (p.fmt_b == FP8_E5M2 ? 1 : 0);
  };
  int shortest[16];
  for (int b = 0; b < 16; ++b) shortest[b] = 0x7FFFFFFF;
  for (int i = 0; i < count; ++i) {
    plan[i] = GroupSlot{eligible(ps[i]) ? 1 : 0, 1, 0, 0};
    if (plan[i].grouped && ps[i].k > 0) {
      const int b = bucket(ps[i]);
      shortest[b] = std::min(shortest[b], ps[i].k / kPipeBK);
    }
  }
  int64_t bytes = 0;
  for (int i = 0; i < count; ++i) {
    if (!plan[i].grouped) continue;
    const GemmProblem& p = ps[i];
    const int nk = p.k / kPipeBK;
    plan[i].kslice = p.k;
    if (nk == 0) continue;
    const int len = std::max(kGroupMinSliceStages, shortest[bucket(p)]);
    int s = std::min(16, std::max(1, nk / len));
    const int per = (nk + s - 1) / s;
    s = (nk + per - 1) / per;
    plan[i].splits = s;
    plan[i].kslice = per * kPipeBK;
    if (s > 1) {
      plan[i].ws_offset = bytes;
      bytes += ((int64_t)s * p.m * p.n * 4 + 255) / 256 * 256;
    }
  }
  return bytes;
}

hipError_t launch_gemm_fwd_group(const GemmProblem* ps, const GroupSlot* plan, const int* idx, int n,
                                 uint8_t* ws, hipStream_t stream) {
  return gemm_detail::launch_group_layout<true, true>(ps, plan, idx, n, ws, stream);
}

}  // namespace fp8lin
