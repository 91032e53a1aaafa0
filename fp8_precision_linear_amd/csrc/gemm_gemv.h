// The forward product for one or two rows whose contraction is a multiple of
// 16 but not of 256 (where it is, the row kernel of gemm_rows.h takes them:
// it streams the weight faster).  Each weight byte is used M <= 2 times, so
// the product is the rate at which W streams from HBM; the tiled kernels fill
// at most 2 of their 128 or 256 tile rows and read W in 64-byte row pieces,
// which reaches ~3 TB/s.  Here every wave reads whole rows of W in 1 KB runs
// (16 contiguous bytes per lane, eight runs in flight), which streams at
// 5-6 TB/s, and forms the dot products on the vector ALU.
//
// "Training and inference of large language models using 8-bit floating
// point", review page, "Proposed method", bullet 3 (the product of the scaled
// FP8 operands, unscaled after the matmul) and bullet 5 (inference).
//
// Arithmetic: every FP8 code converts exactly to fp32 and every product of two
// FP8 values is exact in fp32 (at most 8 significant bits, exponents well
// inside fp32's range).  A lane sums the 16 products of one 1 KB run in a
// chain of fp32 FMAs, adds that to its running sum per output row, and the
// wave adds its 64 lane sums in a fixed butterfly order: the rounding error is
// at most (runs + 21) * 2^-24 * sum |a||b| (recursive summation: 15 for a
// run, one per run added, 6 for the butterfly), 1.7e-6 for K = 8192 and
// 5.1e-6 at the largest K taken (65536), inside the products' 1e-5 bound; the
// same bits on every call.
//
// One workgroup of 16 waves per 16 rows of W: X's M rows are staged in LDS
// once per workgroup (its codes, M * K bytes), then each wave streams its own
// row of W.
//
// Part of gemm_pipe.h (included there after the helpers it uses).
#pragma once

namespace fp8lin {
namespace gemm_detail {

constexpr int kGemvRows = 2;          // output rows at most (see below)
constexpr int kGemvWaves = 16;        // W rows per workgroup (one per wave)
constexpr int kGemvRun = 1024;        // bytes of a W row per wave load (16 per lane)
constexpr int kGemvInFlight = 8;      // runs of a row in flight per wave
constexpr int kGemvLdsBytes = 65536;  // X's codes in LDS at most (M * K)

// The 16 FP8 codes of a lane's run, widened exactly to fp32.
template <int FMT>
__device__ __forceinline__ void gemv_widen(const uint4& c, float (&v)[16]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v2f lo, hi;
    if constexpr (FMT == FP8_E5M2) {
      lo = __builtin_amdgcn_cvt_pk_f32_bf8(w[i], false);
      hi = __builtin_amdgcn_cvt_pk_f32_bf8(w[i], true);
    } else {
      lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
      hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
    }
    v[4 * i] = lo[0];
    v[4 * i + 1] = lo[1];
    v[4 * i + 2] = hi[0];
    v[4 * i + 3] = hi[1];
  }
}

// Y[m][n] = 2^-(ba+bb) * sum_k X[m][k] W[n][k] for m < M <= 2, n in this
// workgroup's 16 rows of W.  A = X [M x K], B = W [N x K], both
// contraction-contiguous, K a multiple of 16 with M * K <= kGemvLdsBytes, rows
// 16-byte aligned (gemv_ok).
template <int FA, int FB, int M, bool ACC>
__global__ __launch_bounds__(kGemvWaves * 64) void gemm_gemv_kernel(GemmProblem p) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kGemvLdsBytes];
  const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
  const int64_t k = p.k;

  // X's rows into LDS (16 bytes per lane and step)
  for (int64_t i = (int64_t)threadIdx.x * 16; i < M * k; i += (int64_t)kGemvWaves * 64 * 16) {
    const int64_t m = i / k, j = i - m * k;
    *reinterpret_cast<uint4*>(xs + i) = *reinterpret_cast<const uint4*>(p.a + m * p.lda + j);
  }
  __syncthreads();

  const int64_t n = (int64_t)blockIdx.x * kGemvWaves + wave;
  if (n >= p.n) return;  // (uniform per wave; no barrier follows)
  const uint8_t* wr = p.b + n * p.ldb;
  const int64_t runs = (k + kGemvRun - 1) / kGemvRun;
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  for (int64_t r0 = 0; r0 < runs; r0 += kGemvInFlight) {
    uint4 wc[kGemvInFlight];
#pragma unroll
    for (int u = 0; u < kGemvInFlight; ++u) {
      const int64_t j = (r0 + u) * kGemvRun + lane * 16;  // this lane's 16 bytes of run r0 + u
      typedef int v4i __attribute__((ext_vector_type(4)));
      v4i t = {0, 0, 0, 0};
      if (j < k) t = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wr + j));
      wc[u] = make_uint4((uint32_t)t[0], (uint32_t)t[1], (uint32_t)t[2], (uint32_t)t[3]);
    }
#pragma unroll
    for (int u = 0; u < kGemvInFlight; ++u) {
      const int64_t j = (r0 + u) * kGemvRun + lane * 16;
      if (r0 + u >= runs) break;  // (uniform)
      float wv[16];
      gemv_widen<FB>(wc[u], wv);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4 xc = j < k ? *reinterpret_cast<const uint4*>(xs + m * k + j) : make_uint4(0u, 0u, 0u, 0u);
        float xv[16];
        gemv_widen<FA>(xc, xv);
        float t = wv[0] * xv[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) t = __builtin_fmaf(wv[i], xv[i], t);
        acc[m] += t;
      }
    }
  }

  const int unscale = -(*p.bias_a + *p.bias_b);
  uint32_t mx = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float s = acc[m];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) {
      float* c = p.c + (int64_t)m * p.ldc + n;
      float v = __builtin_ldexpf(s, unscale);
      if constexpr (ACC) v = *c + v;
      *c = v;
      mx = max(mx, __float_as_uint(v) & 0x7FFFFFFFu);
    }
  }
  if (p.amax) amax_fold(mx, p.amax);
}

// Whether a product takes the vector kernel: the forward layout (both
// operands contraction-contiguous), exact arithmetic, one or two output rows,
// a contraction that is a multiple of 16 and whose X rows fit the LDS, 16-byte
// aligned rows, fewer than 2^26 columns.
template <bool AK, bool BK>
bool gemv_ok(const GemmProblem& p) {
  if constexpr (!(AK && BK)) {
    return false;
  } else {
    if (p.math == kMathNativeFp8 || p.m < 1 || p.m > kGemvRows || p.n < 1) return false;
    if (p.k % 16 != 0 || (int64_t)p.m * p.k > kGemvLdsBytes) return false;
    // a dispatch counts its lanes in 32 bits: 1024 per 16 columns
    if ((int64_t)((p.n + kGemvWaves - 1) / kGemvWaves) * (kGemvWaves * 64) > (int64_t)0xFFFFFFFF) return false;
    auto aligned = [](const void* q, int64_t ld) { return ((uintptr_t)q % 16 == 0) && (ld % 16 == 0); };
    return aligned(p.a, p.lda) && aligned(p.b, p.ldb);
  }
}

template <int M, bool ACC>
hipError_t launch_gemv_rows(const GemmProblem& p, hipStream_t stream) {
  const dim3 grid((uint32_t)((p.n + kGemvWaves - 1) / kGemvWaves)), block(kGemvWaves * 64);
#define FP8LIN_GEMV_CASE(FA, FB)                                                                        \
  if (p.fmt_a == FA && p.fmt_b == FB) {                                                                 \
    hipLaunchKernelGGL((gemm_gemv_kernel<FA, FB, M, ACC>), grid, block, 0, stream, p);                \
    return hipGetLastError();                                                                           \
  }
  FP8LIN_GEMV_CASE(FP8_E4M3, FP8_E4M3)
  FP8LIN_GEMV_CASE(FP8_E5M2, FP8_E4M3)
  FP8LIN_GEMV_CASE(FP8_E4M3, FP8_E5M2)
  FP8LIN_GEMV_CASE(FP8_E5M2, FP8_E5M2)
#undef FP8LIN_GEMV_CASE
  return hipErrorInvalidValue;
}

template <int M>
hipError_t launch_gemv_m(const GemmProblem& p, hipStream_t stream) {
  return p.accumulate ? launch_gemv_rows<M, true>(p, stream) : launch_gemv_rows<M, false>(p, stream);
}

// One or two rows only: the FMAs grow with the rows and the vector ALU, not
// HBM, bounds three or more (28672 x 8192 weights: 38.1, 46.2, 68.7 and
// 79.9 us for 1 to 4 rows, against ~72 us in the tiled kernels and 37 us in
// the row kernel).
inline hipError_t launch_gemv(const GemmProblem& p, hipStream_t stream) {
  return p.m == 1 ? launch_gemv_m<1>(p, stream) : launch_gemv_m<2>(p, stream);
}

}  // namespace gemm_detail
}  // namespace fp8lin
