// Products split along the contraction, for outputs of too few 128x128 tiles
// to occupy the chip's 256 workgroup slots (a small batch of tokens, or an
// output with a short side): `splits` blocks per output tile, block s summing
// the contraction slice [s * kslice, min(k, (s + 1) * kslice)) with the
// 128x128 pipelined kernel's main loop and storing its raw sum (not unscaled)
// in a caller-provided workspace, slice s at ws + s * m * n (row-major m x n).
// A second kernel then adds the slices in slice order and unscales once by
// 2^-(bias_a + bias_b), so the result does not depend on timing: the same
// inputs give the same bits on every call.
#pragma once

#include "gemm_pipe.h"

namespace fp8lin {
namespace gemm_detail {

// How a product is split: splits == 1 means not at all.
struct SplitPlan {
  int splits;
  int kslice;  // contraction bytes per slice (a multiple of kPipeBK)
};

// Each slice at least 24 stages (1536 contraction bytes): the slices' sums
// then outweigh the extra pass that adds them.  Measured on MI355X, split in
// two against unsplit: 2048 x 768 outputs with contractions of 48 stages
// 1.10-1.12x faster, of 36 stages 0.97x, a 2304 x 768 output of 32 stages
// 0.93x; 128-row outputs of 128 and 448 stages split in four 1.9x and 2.8x.
constexpr int kSplitMinStages = 24;
constexpr int kSplitSlots = 256;    // workgroups the chip runs at once (one per CU)

// FP8LIN_SPLIT_SLOTS overrides kSplitSlots (tuning).
inline int64_t split_slots() {
  const char* v = std::getenv("FP8LIN_SPLIT_SLOTS");
  const int64_t s = v ? std::atoll(v) : kSplitSlots;
  return s < 1 ? 1 : s;
}

// The split for an m x n output with contraction k, each slice at least
// kSplitMinStages stages; none when the contraction is not a whole number of
// stages (those products run the general kernel).  Two candidates: as many
// slices as leave one workgroup per CU beside the output's 128x128 tiles, and
// as many as leave two.  Each is costed in stage times of a workgroup alone
// on a CU (~0.5 us: 10240 x 8192 at 192 rows, 160 workgroups of 128 stages,
// 63.5 us): the busiest CU's stages (ceil(W / slots) workgroups of nk / s
// stages, W = tiles x s), divided by 1.15 where two workgroups share a CU
// (one's LDS reads and conversions run under the other's MFMAs: 8192 x 28672
// at 65 rows, 112 stages per CU as four or eight slices, 71.2 against 62.6
// us), plus the pass that adds the slices ((s + 1) x m x n x 4 bytes at
// ~5 TB/s).  On 20 outputs of 65-384 rows through 70B weights this takes the
// faster plan, up to 27% faster than one workgroup per CU alone (10240 x 8192
// at 192 rows: three slices 49.9 us, unsplit 63.2), and keeps plans the
// second candidate would slow (8192 x 8192 at 128 rows: four slices 27.2,
// five 30.6).  The second candidate is taken only if its workspace fits
// max_bytes; the first needs at most slots x 64 KiB (16 MiB).
inline SplitPlan plan_split(int64_t m, int64_t n, int64_t k, int64_t max_bytes = INT64_MAX) {
  if (m <= 0 || n <= 0 || k <= 0 || k % kPipeBK != 0) return SplitPlan{1, 0};
  const int64_t tiles = ((m + 127) / 128) * ((n + 127) / 128);
  const int64_t nk = k / kPipeBK, smax = nk / kSplitMinStages, slots = split_slots();
  auto clamp = [&](int64_t v) { return v < smax ? v : smax; };
  auto cost = [&](int64_t v) {
    const int64_t per_cu = (tiles * v + slots - 1) / slots;
    const double reduce = v > 1 ? (double)(v + 1) * (double)m * (double)n * 4.0 / 2.5e6 : 0.0;
    return (double)per_cu * (double)nk / (double)v / (per_cu > 1 ? 1.15 : 1.0) + reduce;
  };
  int64_t s = clamp(slots / tiles);
  const int64_t s2 = clamp(2 * slots / tiles);
  if (s2 > s && s2 >= 2 && cost(s2) < cost(s < 1 ? 1 : s) - 1e-9 && s2 * m * n * 4 <= max_bytes) s = s2;
  if (s < 2) return SplitPlan{1, 0};
  const int64_t per = (nk + s - 1) / s;  // stages per slice; the last may be shorter
  return SplitPlan{(int)((nk + per - 1) / per), (int)(per * kPipeBK)};
}

inline int64_t split_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t max_bytes = INT64_MAX) {
  const SplitPlan sp = plan_split(m, n, k, max_bytes);
  return sp.splits > 1 ? (int64_t)sp.splits * m * n * 4 : 0;
}

// Store a wave's TM x TN block of 32x32 accumulator tiles as they are (no
// unscale) into the m x n slice c, bounds-checked.  Accumulator layout as in
// store_block_as.
template <int TM, int TN>
__device__ __forceinline__ void store_raw_block(float* c, int m, int n, const v16f (&acc)[TM][TN],
                                                int row0, int col0, int lane) {
  const int h = lane >> 5, rl = lane & 31;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = col0 + j * 32 + rl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < m && col < n) c[(int64_t)row * n + col] = acc[i][j][r];
      }
    }
}

// Block b: slice b / tiles, output tile b % tiles (ordered as tile_coords
// orders a 128x128 launch).
template <bool AK, bool BK, int FA, int FB, int MATH>
__global__ __launch_bounds__(256) void gemm_quad_split_kernel(GemmProblem p, int tiles_m, int tiles_n,
                                                              int kslice, float* ws) {
  constexpr int R = 128;
  __shared__ __attribute__((aligned(1024))) uint8_t sa[kPipeStages * R * kPipeBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sb[kPipeStages * R * kPipeBK];

  const int tiles = tiles_m * tiles_n;
  const int s = (int)blockIdx.x / tiles;
  int tm, tn;
  tile_coords((int)blockIdx.x - s * tiles, tiles_m, tiles_n, tm, tn);
  const int lane = (int)threadIdx.x & 63, wave = wave_id();
  const int m0 = tm * R, n0 = tn * R;

  // the slice: contraction [k0, k0 + q.k) of both operands
  const int k0 = s * kslice;
  GemmProblem q = p;
  q.k = min(kslice, p.k - k0);
  q.a = p.a + (AK ? (int64_t)k0 : (int64_t)k0 * p.lda);
  q.b = p.b + (BK ? (int64_t)k0 : (int64_t)k0 * p.ldb);

  v16f acc[2][2];
  zero_acc(acc);
  QuadWave<AK, BK, FA, FB, MATH> w(q, m0, n0, wave, lane, lds_addr(sa), lds_addr(sb), acc);
  w.run();
  store_raw_block(ws + (int64_t)s * p.m * p.n, p.m, p.n, acc, m0 + (wave >> 1) * (R / 2),
                  n0 + (wave & 1) * (R / 2), lane);
}

// out[i] = 2^-(bias_a + bias_b) * sum over s = 0, 1, ... of ws[s * mn + i],
// in that order; out is the contiguous m x n output.  VEC: four elements per
// lane (mn a multiple of 4, so every slice starts 16-byte aligned).
constexpr int kReduceThreads = 256;

template <bool VEC>
__global__ __launch_bounds__(kReduceThreads) void split_reduce_kernel(const float* __restrict__ ws,
                                                                      int splits, int64_t mn,
                                                                      const int32_t* bias_a,
                                                                      const int32_t* bias_b,
                                                                      float* __restrict__ out) {
  const int unscale = -(*bias_a + *bias_b);
  const int64_t stride = (int64_t)gridDim.x * kReduceThreads;
  const int64_t first = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x;
  if constexpr (VEC) {
    const int64_t n4 = mn / 4;
    const float4* w4 = reinterpret_cast<const float4*>(ws);
    float4* o4 = reinterpret_cast<float4*>(out);
    for (int64_t i = first; i < n4; i += stride) {
      float4 acc = w4[i];
      for (int s = 1; s < splits; ++s) {
        const float4 v = w4[(int64_t)s * n4 + i];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
      o4[i] = make_float4(__builtin_ldexpf(acc.x, unscale), __builtin_ldexpf(acc.y, unscale),
                          __builtin_ldexpf(acc.z, unscale), __builtin_ldexpf(acc.w, unscale));
    }
  } else {
    for (int64_t i = first; i < mn; i += stride) {
      float acc = ws[i];
      for (int s = 1; s < splits; ++s) acc += ws[(int64_t)s * mn + i];
      out[i] = __builtin_ldexpf(acc, unscale);
    }
  }
}

template <bool AK, bool BK, int MATH>
hipError_t launch_split_math(const GemmProblem& p, const SplitPlan& sp, float* ws, hipStream_t stream) {
  int tiles_m, tiles_n;
  tile_grid(p, 128, 128, tiles_m, tiles_n);
  const dim3 grid((uint32_t)(tiles_m * tiles_n * sp.splits)), block(256);
#define FP8LIN_SPLIT_CASE(FA, FB)                                                                  \
  if (p.fmt_a == FA && p.fmt_b == FB) {                                                            \
    hipLaunchKernelGGL((gemm_quad_split_kernel<AK, BK, FA, FB, MATH>), grid, block, 0, stream, p, \
                       tiles_m, tiles_n, sp.kslice, ws);                                           \
  } else
  FP8LIN_SPLIT_CASE(FP8_E4M3, FP8_E4M3)
  FP8LIN_SPLIT_CASE(FP8_E5M2, FP8_E4M3)
  FP8LIN_SPLIT_CASE(FP8_E4M3, FP8_E5M2)
  FP8LIN_SPLIT_CASE(FP8_E5M2, FP8_E5M2)
  return hipErrorInvalidValue;
#undef FP8LIN_SPLIT_CASE
  if (hipError_t e = hipGetLastError()) return e;
  const int64_t mn = (int64_t)p.m * p.n;
  const int64_t units = (mn & 3) == 0 ? mn / 4 : mn;
  int64_t blocks = (units + kReduceThreads - 1) / kReduceThreads;
  blocks = blocks < 1 ? 1 : (blocks > 8192 ? 8192 : blocks);
  if ((mn & 3) == 0)
    hipLaunchKernelGGL(split_reduce_kernel<true>, dim3((uint32_t)blocks), dim3(kReduceThreads), 0, stream,
                       ws, sp.splits, mn, p.bias_a, p.bias_b, p.c);
  else
    hipLaunchKernelGGL(split_reduce_kernel<false>, dim3((uint32_t)blocks), dim3(kReduceThreads), 0, stream,
                       ws, sp.splits, mn, p.bias_a, p.bias_b, p.c);
  return hipGetLastError();
}

// The product with a workspace: split when the plan (within max_bytes of
// workspace) says so and the pipelined kernels take the operands (ws holds at
// least split_workspace_bytes with the same max_bytes), otherwise exactly
// launch_layout.  The output must be contiguous (ldc == n).  A forward
// product of at most 64 rows (two at most when K is not a multiple of 256)
// takes the small-row kernels instead (gemm_gemv.h, gemm_rows.h; the
// workspace goes unused).
template <bool AK, bool BK>
hipError_t launch_layout_ws(const GemmProblem& p, float* ws, int64_t max_bytes, hipStream_t stream) {
  const SplitPlan sp = plan_split(p.m, p.n, p.k, max_bytes);
  if (sp.splits <= 1 || !pipe_ok<AK, BK>(p) || p.ldc != p.n || p.amax || gemv_ok<AK, BK>(p) ||
      rows_ok<AK, BK>(p))
    return launch_layout<AK, BK>(p, stream);
  if (p.math == kMathNativeFp8) return launch_split_math<AK, BK, kMathNativeFp8>(p, sp, ws, stream);
  if (exact_on_bf16(p)) return launch_split_math<AK, BK, kMathExactBf16>(p, sp, ws, stream);
  return launch_split_math<AK, BK, kMathExact>(p, sp, ws, stream);
}

}  // namespace gemm_detail
}  // namespace fp8lin
