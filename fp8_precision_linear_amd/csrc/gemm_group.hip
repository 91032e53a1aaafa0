// The products of a training step in one launch: the forward product
// (E4M3 x E4M3, both operands contraction-contiguous, fp16 MFMA), the data
// gradient (E5M2 x E4M3, bf16 MFMA) and the weight gradient (E5M2 x E4M3,
// bf16 MFMA) -- "Proposed method", bullets 3-5 -- of any number of layers,
// as blocks of one grid (each block's entry names which of the three it is).
// The GPU then balances all of them together: a launch per operand layout
// ends with a part-empty wave each.  Split products' slices are added by one
// reduction launch for all of them.  Other format pairs and layouts run per
// layout (gemm_group.h).
#include <algorithm>

#include "gemm_group.h"

namespace fp8lin {
namespace gemm_detail {
namespace {

// The training-step variants and their kernels' template arguments.
constexpr int kVarFwd = 0, kVarDgrad = 1, kVarWgrad = 2;

template <int MATH_FWD, int MATH_GRAD>
__global__ __launch_bounds__(256) void gemm_step_kernel(GroupArgs args) {
  __shared__ __attribute__((aligned(1024))) uint8_t sa[kPipeStages * 128 * kPipeBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sb[kPipeStages * 128 * kPipeBK];
  const auto* e = group_entry<GroupArgs, GroupEntry>();
  switch (e->variant) {
    case kVarFwd: group_block<true, true, FP8_E4M3, FP8_E4M3, MATH_FWD>(e, sa, sb); break;
    case kVarDgrad: group_block<true, false, FP8_E5M2, FP8_E4M3, MATH_GRAD>(e, sa, sb); break;
    default: group_block<false, false, FP8_E5M2, FP8_E4M3, MATH_GRAD>(e, sa, sb); break;
  }
}

}  // namespace

// The variant of a product in the training-step kernel, or -1: its layout and
// formats must be one of the three, and its exact arithmetic the MFMA the
// kernel uses for it (the tuning override FP8LIN_EXACT_MFMA may say
// otherwise).
int step_variant(const GemmProblem& p) {
  int v = -1;
  if (p.a_kmajor && p.b_kmajor && p.fmt_a == FP8_E4M3 && p.fmt_b == FP8_E4M3) v = kVarFwd;
  else if (p.a_kmajor && !p.b_kmajor && p.fmt_a == FP8_E5M2 && p.fmt_b == FP8_E4M3) v = kVarDgrad;
  else if (!p.a_kmajor && !p.b_kmajor && p.fmt_a == FP8_E5M2 && p.fmt_b == FP8_E4M3) v = kVarWgrad;
  if (v < 0 || p.math == kMathNativeFp8) return v;
  return exact_on_bf16(p) == (v != kVarFwd) ? v : -1;
}

}  // namespace gemm_detail

int gemm_step_variant(const GemmProblem& p) { return gemm_detail::step_variant(p); }

hipError_t launch_gemm_step_group(const GemmProblem* ps, const GroupSlot* plan, const int* idx_in, int n,
                                  uint8_t* ws, hipStream_t stream) {
  using namespace gemm_detail;
  int idx[kGroupMaxProducts];
  for (int j = 0; j < n; ++j) idx[j] = idx_in[j];
  order_longest_first(plan, idx, n);
  for (int lo = 0; lo < n; lo += kGroupMax) {
    const int cnt = n - lo < kGroupMax ? n - lo : kGroupMax;
    GroupArgs g{};
    ReduceArgs r{};
    g.count = cnt;
    int64_t blocks = 0, rblocks = 0;
    for (int j = 0; j < cnt; ++j) {
      const GemmProblem& p = ps[idx[lo + j]];
      const GroupSlot& sl = plan[idx[lo + j]];
      GroupEntry& e = g.e[j];
      e.p = p;
      e.p.amax = nullptr;
      e.tiles_m = (p.m + 127) / 128;
      e.tiles_n = (p.n + 127) / 128;
      e.splits = sl.splits;
      e.kslice = sl.kslice;
      e.first = (int)blocks;
      e.variant = step_variant(p);
      e.ws = sl.splits > 1 ? reinterpret_cast<float*>(ws + sl.ws_offset) : nullptr;
      blocks += (int64_t)e.tiles_m * e.tiles_n * e.splits;
      if (sl.splits > 1) {
        ReduceEntry& q = r.e[r.count++];
        const int64_t mn = (int64_t)p.m * p.n;
        const bool vec = (mn & 3) == 0;
        const int64_t units = vec ? mn / 4 : mn;
        int64_t b = (units + kReduceThreads - 1) / kReduceThreads;
        b = b < 1 ? 1 : (b > 2048 ? 2048 : b);
        q = ReduceEntry{e.ws, p.c, p.bias_a, p.bias_b, mn, sl.splits, (int)rblocks, (int)b, vec ? 1 : 0};
        rblocks += b;
      }
    }
    if (ps[idx[lo]].math == kMathNativeFp8)
      hipLaunchKernelGGL((gemm_step_kernel<kMathNativeFp8, kMathNativeFp8>), dim3((uint32_t)blocks), dim3(256),
                         0, stream, g);
    else
      hipLaunchKernelGGL((gemm_step_kernel<kMathExact, kMathExactBf16>), dim3((uint32_t)blocks), dim3(256), 0,
                         stream, g);
    if (hipError_t err = hipGetLastError()) return err;
    if (r.count > 0) {
      hipLaunchKernelGGL(group_reduce_kernel<0>, dim3((uint32_t)rblocks), dim3(kReduceThreads), 0, stream, r);
      if (hipError_t err = hipGetLastError()) return err;
    }
  }
  return hipSuccess;
}

}  // namespace fp8lin
