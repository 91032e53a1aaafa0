// FP8 product kernels, forward: both operands contraction-contiguous.
// One translation unit per operand layout so the instantiations compile in parallel.
#include <algorithm>

#include "gemm_group.h"

namespace fp8lin {

hipError_t launch_gemm_fwd(const GemmProblem& p, hipStream_t stream) {
  return gemm_detail::launch_layout<true, true>(p, stream);
}

hipError_t launch_gemm_fwd_ws(const GemmProblem& p, float* ws, int64_t max_bytes, hipStream_t stream) {
  return gemm_detail::launch_layout_ws<true, true>(p, ws, max_bytes, stream);
}

int64_t gemm_split_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t max_bytes) {
  return gemm_detail::split_workspace_bytes(m, n, k, max_bytes);
}

// Which products run grouped and how they are split.  The training-step
// products (forward E4M3 x E4M3, data and weight gradients E5M2 x E4M3) share
// one launch; any other product is launched with those of its layout and
// format pair.  A launch's blocks are handed out in order as workgroup slots
// free up (kGroupSlots of them: two 128 x 128 workgroups per CU), and its
// launcher orders products longest first, so the work balances without
// splitting as long as no single block holds more than the average work per
// slot: a product is cut along the contraction only into slices of at least
// that average (and at least kGroupMinSliceStages stages, at most 16 slices)
// -- which happens when a launch has too few tiles to fill the slots.
// A forward product of few rows through a weight of 16 MiB or more runs alone
// in a small-row kernel (gemm_rows.h, gemm_gemv.h), which streams the weight
// at 5-7 TB/s where a grouped launch's 128 x 128 tiles reach about 3.
int64_t gemm_group_plan(const GemmProblem* ps, int count, GroupSlot* plan) {
  using namespace gemm_detail;
  auto eligible = [](const GemmProblem& p) {
    if (p.m <= 0 || p.n <= 0 || p.ldc != p.n) return false;
    const int64_t tiles = (int64_t)((p.m + 127) / 128) * ((p.n + 127) / 128);
    if (tiles >= kGroupMaxTiles) return false;
    if (p.a_kmajor && p.b_kmajor && (int64_t)p.n * p.k >= ((int64_t)1 << 24) &&
        (rows_ok<true, true>(p) || gemv_ok<true, true>(p)))
      return false;
    if (p.a_kmajor && p.b_kmajor) return pipe_ok<true, true>(p);
    if (p.a_kmajor && !p.b_kmajor) return pipe_ok<true, false>(p);
    if (!p.a_kmajor && !p.b_kmajor) return pipe_ok<false, false>(p);
    return false;
  };
  // launch groups: the training-step products (key 16), else one per layout
  // and format pair
  auto bucket = [](const GemmProblem& p) {
    if (gemm_step_variant(p) >= 0) return 16;
    return (p.a_kmajor ? 1 : 0) + (p.b_kmajor ? 2 : 0) + 4 * (p.fmt_a == FP8_E5M2 ? 1 : 0) +
           8 * (p.fmt_b == FP8_E5M2 ? 1 : 0);
  };
  int64_t work[17] = {0};  // tile-stages of each launch group
  for (int i = 0; i < count; ++i) {
    plan[i] = GroupSlot{eligible(ps[i]) ? 1 : 0, 1, ps[i].k, 0};
    if (plan[i].grouped) {
      const GemmProblem& p = ps[i];
      work[bucket(p)] += (int64_t)((p.m + 127) / 128) * ((p.n + 127) / 128) * (p.k / kPipeBK);
    }
  }
  int64_t bytes = 0;
  for (int i = 0; i < count; ++i) {
    if (!plan[i].grouped) continue;
    const GemmProblem& p = ps[i];
    const int nk = p.k / kPipeBK;
    if (nk == 0) continue;
    const int64_t avg = (work[bucket(p)] + kGroupSlots - 1) / kGroupSlots;
    const int len = (int)std::max<int64_t>(kGroupMinSliceStages, avg);
    int s = std::min(16, (nk + len - 1) / len);
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
