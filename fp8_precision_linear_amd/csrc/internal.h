// Internal declarations shared by the HIP translation units of libfp8lin.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8lin.h"

namespace fp8lin {

// Quantisation kernels (quant.hip).
hipError_t launch_amax(const void* x, int dtype, int64_t n, float* amax, hipStream_t stream);
hipError_t launch_bias(const float* amax, int fmt, int32_t margin, int32_t* bias,
                       hipStream_t stream);
// amax: optional; when given, cleared, then max |x| (fp32 bits) folded in.
hipError_t launch_cast(const void* x, int dtype, int64_t n, const int32_t* bias, int fmt,
                       uint8_t* y, uint32_t* amax, hipStream_t stream);
// *p = 0 (one lane).
hipError_t launch_clear_u32(uint32_t* p, hipStream_t stream);
// amax -> bias -> cast of one tensor, results bit-identical to launch_amax,
// launch_bias and launch_cast in turn: one launch for small tensors, three
// (clear, amax, a cast that derives the bias itself) for the rest.
hipError_t launch_quantize(const void* x, int dtype, int64_t n, int fmt, int32_t margin, uint8_t* y,
                           float* amax, int32_t* bias, hipStream_t stream);

// Delayed scaling in one call (fp8_quantize_delayed): the bias from the amax
// word (the previous step's), the cast, then max |x| of this input into the
// same word; two launches (one for small tensors).
hipError_t launch_quantize_delayed(const void* x, int dtype, int64_t n, int fmt, int32_t margin,
                                   uint8_t* y, float* amax, int32_t* bias, hipStream_t stream);

// The quantisation of several tensors (fp8_quantize_multi): one launch per 32
// small tensors (one workgroup each), three launches per 32 others; every
// tensor's results those of launch_quantize on it alone.
struct QuantDesc {
  const void* x;
  int64_t n;
  int dtype, fmt;
  int32_t margin;
  uint8_t* y;
  float* amax;
  int32_t* bias;
};
hipError_t launch_quantize_multi(const QuantDesc* d, int count, hipStream_t stream);

// SwiGLU between the products of a chained MLP (swiglu.hip).  amax: optional,
// cleared then folded with max |output| (fp32 magnitude bits).
hipError_t launch_swiglu_fwd(const float* h, int64_t rows, int64_t f, uint16_t* a, uint32_t* amax,
                             hipStream_t stream);
hipError_t launch_swiglu_bwd(const float* h, const float* da, int64_t rows, int64_t f, uint16_t* dh,
                             uint32_t* amax, hipStream_t stream);
// Blocks the SwiGLU launches use for a rows x f output (must fit a 32-bit grid).
int64_t swiglu_blocks(int64_t rows, int64_t f);

// Product arithmetic (the values of fp8_scaled_gemm's `math` argument).
#define FP8LIN_MATH_EXACT FP8_GEMM_EXACT
#define FP8LIN_MATH_NATIVE_FP8 FP8_GEMM_NATIVE_FP8

// One FP8 product C[m][n] = 2^-(*bias_a + *bias_b) * sum_k A(m, k) * B(k, n).
// A(m, k) lives at a[m * lda + k] when a_kmajor, else at a[k * lda + m];
// B(k, n) lives at b[n * ldb + k] when b_kmajor, else at b[k * ldb + n].
struct GemmProblem {
  const uint8_t* a;
  int64_t lda;
  bool a_kmajor;
  int fmt_a;
  const int32_t* bias_a;
  const uint8_t* b;
  int64_t ldb;
  bool b_kmajor;
  int fmt_b;
  const int32_t* bias_b;
  float* c;
  int64_t ldc;
  int m, n, k;
  int math;
  // optional: fold max |C[m][n]| (as fp32 magnitude bits) into *amax with
  // atomicMax; nullptr for none
  uint32_t* amax;
  // C[m][n] += the unscaled product (one fp32 addition per output) instead
  // of C[m][n] = it; only the single-product kernels (pipelined and general)
  // take it
  bool accumulate;
};

// One launcher per operand layout (gemm_fwd.hip, gemm_dgrad.hip, gemm_wgrad.hip).
hipError_t launch_gemm_fwd(const GemmProblem& p, hipStream_t stream);    // A, B contraction-contiguous
hipError_t launch_gemm_dgrad(const GemmProblem& p, hipStream_t stream);  // B contraction-strided
hipError_t launch_gemm_wgrad(const GemmProblem& p, hipStream_t stream);  // A, B contraction-strided
// The same with a workspace (gemm_split.h): an output of too few 128x128 tiles
// to fill the chip is computed split along the contraction, the slices' raw
// sums in ws, then added in slice order and unscaled.  The split is planned
// within max_bytes of workspace; ws holds at least
// gemm_split_workspace_bytes(p.m, p.n, p.k, max_bytes) bytes, 16-byte
// aligned; the output must be contiguous.  Anything not split runs as
// launch_gemm_*.
hipError_t launch_gemm_fwd_ws(const GemmProblem& p, float* ws, int64_t max_bytes, hipStream_t stream);
hipError_t launch_gemm_dgrad_ws(const GemmProblem& p, float* ws, int64_t max_bytes, hipStream_t stream);
hipError_t launch_gemm_wgrad_ws(const GemmProblem& p, float* ws, int64_t max_bytes, hipStream_t stream);
// Workspace bytes the split of an m x n output with contraction k needs,
// planned within max_bytes where it can be (0: not split; more than max_bytes
// only where even the one-workgroup-per-CU split needs more).
int64_t gemm_split_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t max_bytes);

// Several products run together (fp8_scaled_gemm_group, gemm_group.h).
constexpr int kGroupMaxProducts = 256;  // products per call
struct GroupSlot {
  int grouped;        // 1: in a grouped launch; 0: launched on its own
  int splits;         // contraction slices (1: not split)
  int kslice;         // contraction bytes per slice
  int64_t ws_offset;  // splits > 1: the slices' bytes in the workspace start here
};
// The plan of count products (ps: every output contiguous, ldc == n); returns
// the workspace bytes it needs.
int64_t gemm_group_plan(const GemmProblem* ps, int count, GroupSlot* plan);
// The grouped products ps[idx[0..n)] of one operand layout each.
hipError_t launch_gemm_fwd_group(const GemmProblem* ps, const GroupSlot* plan, const int* idx, int n,
                                 uint8_t* ws, hipStream_t stream);
hipError_t launch_gemm_dgrad_group(const GemmProblem* ps, const GroupSlot* plan, const int* idx, int n,
                                   uint8_t* ws, hipStream_t stream);
hipError_t launch_gemm_wgrad_group(const GemmProblem* ps, const GroupSlot* plan, const int* idx, int n,
                                   uint8_t* ws, hipStream_t stream);
// The training-step products (forward E4M3 x E4M3, data and weight gradients
// E5M2 x E4M3, each on the MFMA its single launch would use) in one launch
// (gemm_group.hip); gemm_step_variant is -1 for any other product.
int gemm_step_variant(const GemmProblem& p);
hipError_t launch_gemm_step_group(const GemmProblem* ps, const GroupSlot* plan, const int* idx, int n,
                                  uint8_t* ws, hipStream_t stream);

}  // namespace fp8lin
