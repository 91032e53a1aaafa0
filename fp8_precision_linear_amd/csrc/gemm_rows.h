// The forward product for 3 to 32 rows (a few tokens through a large weight,
// as when a served model decodes a small batch).  The weight streams from HBM
// once; the tiled kernels read it in 64-byte pieces of 16 rows per load and
// reach ~3 TB/s there.  Here the weight's rows arrive through LDS DMA in 256-byte
// runs (each load covers four rows x 256 contiguous bytes), and the products run
// on the exact 16-bit MFMA as in the tiled kernels.
//
// "Training and inference of large language models using 8-bit floating
// point", review page, "Proposed method", bullet 3 (the product of the scaled
// FP8 operands, unscaled after the matmul) and bullet 5 (inference).
//
// One workgroup of eight waves per 32 output columns (32 rows of W) and all M
// rows.  Stage = 256 contraction bytes: a 32 x 256-byte tile of W and one of X
// (X's rows past M re-read row M - 1 and are zeroed in the fragments), four
// stages in a ring, three in flight.  Wave w multiplies bytes [32w, 32w + 32)
// of every stage (two 32x32x16 MFMAs) into its own 32x32 partial sum; the
// eight partial sums meet in LDS and are added in wave order (the same bits on
// every call), then unscaled once.  Exact arithmetic only: the native FP8
// path keeps the tiled kernels, whose 64-product groups its error bound
// assumes.
//
// Part of gemm_pipe.h (included there after the helpers it uses).
#pragma once

namespace fp8lin {
namespace gemm_detail {

constexpr int kRowsMin = 3, kRowsMax = 32;  // output rows taken (1 and 2: gemm_gemv.h)
constexpr int kRowsStage = 256;             // contraction bytes per stage
constexpr int kRowsTile = 32 * kRowsStage;  // one operand's stage tile (8 KB)
constexpr int kRowsWaves = 8;

// Physical 16-byte chunk of logical chunk c in row r of a stage tile: the 16
// rows that 16 lanes of one fragment read then fall in 16 different bank
// groups (a row is one 256-byte bank window).
__device__ __forceinline__ int rows_swz(int r, int c) { return c ^ (r & 15); }

// Stage s of rows [r0, r0 + 32) of an operand (row length ld) into the stage
// tile at LDS address `tile`: KB q (this wave's: q = wave) holds rows
// 4q .. 4q + 3; lane l lands at row 4q + l / 16, physical chunk l % 16, and
// fetches the logical chunk that maps there.  Rows past `rows` re-read row
// rows - 1.
__device__ __forceinline__ void rows_dma(const uint8_t* base, int64_t ld, int r0, int rows, int s, uint32_t tile,
                                         int wave, int lane) {
  const int r = 4 * wave + (lane >> 4), pc = lane & 15;
  const int lc = rows_swz(r, pc);  // the XOR is its own inverse
  const int gr = min(r0 + r, rows - 1);
  dma16(base + (int64_t)gr * ld + (int64_t)s * kRowsStage + 16 * lc, tile + wave * 1024);
}

template <int FA, int FB, int MATH, bool ACC>
__global__ __launch_bounds__(kRowsWaves * 64) void gemm_rows_kernel(GemmProblem p) {
  // ring of four stages: slot s holds W's tile at 2 s * 8 KB and X's after it;
  // at the end it holds the eight waves' partial sums (32 KB)
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kPipeStages * 2 * kRowsTile];
  const int lane = (int)threadIdx.x & 63, wave = wave_id();
  const int rl = lane & 31, h = lane >> 5;
  const int n0 = (int)blockIdx.x * 32;
  const uint32_t ring0 = lds_addr(ring);
  const int nk = p.k / kRowsStage;
  auto issue = [&](int s, int slot) {
    const uint32_t t = ring0 + slot * 2 * kRowsTile;
    rows_dma(p.b, p.ldb, n0, p.n, s, t, wave, lane);
    rows_dma(p.a, p.lda, 0, p.m, s, t + kRowsTile, wave, lane);
  };
  // this lane's fragment: logical chunk 2 wave + h of row rl
  const uint32_t frag = rl * kRowsStage + (rows_swz(rl, 2 * wave + h) << 4);
  const bool xrow = rl < p.m;

  v16f acc[1][1];
  zero_acc(acc);
#pragma unroll
  for (int s = 0; s < 3; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt & 3;
    wait_stages<2>(min(2, nk - 1 - kt));
    bare_barrier();
    if (kt + 3 < nk) issue(kt + 3, (kt + 3) & 3);
    typedef int v4i __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const v4i* lds_v4i;
    const uint32_t t = ring0 + slot * 2 * kRowsTile + opaque(frag);
    const v4i w = *(lds_v4i)(uintptr_t)t;
    v4i x = *(lds_v4i)(uintptr_t)(t + kRowsTile);
    if (!xrow) x = v4i{0, 0, 0, 0};
    // two 32x32x16 steps over the lane's 16 bytes (8 contraction values each)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if constexpr (MATH == kMathExactBf16) {
        const v8bf a = fp8x8_to_bf16<FA>(x[2 * q], x[2 * q + 1]);
        const v8bf b = fp8x8_to_bf16<FB>(w[2 * q], w[2 * q + 1]);
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[0][0], 0, 0, 0);
      } else {
        const v8h a = fp8x8_to_f16<FA>(x[2 * q], x[2 * q + 1]);
        const v8h b = fp8x8_to_f16<FB>(w[2 * q], w[2 * q + 1]);
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[0][0], 0, 0, 0);
      }
    }
  }

  // every wave's LDS reads are done (their values fed the MFMAs) and no DMA
  // is in flight (the last stage was waited for): the ring takes the partial
  // sums.  32x32 accumulator layout: register r of lane l holds row
  // 8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32.
  __syncthreads();
  float (*part)[32][32] = reinterpret_cast<float (*)[32][32]>(ring);
#pragma unroll
  for (int r = 0; r < 16; ++r) part[wave][8 * (r >> 2) + 4 * h + (r & 3)][rl] = acc[0][0][r];
  __syncthreads();

  const int unscale = -(*p.bias_a + *p.bias_b);
  uint32_t mx = 0;
#pragma unroll
  for (int o = (int)threadIdx.x; o < 32 * 32; o += kRowsWaves * 64) {
    const int row = o / 32, col = o % 32;
    float sum = part[0][row][col];
#pragma unroll
    for (int w2 = 1; w2 < kRowsWaves; ++w2) sum += part[w2][row][col];
    if (row < p.m && n0 + col < p.n) {
      float* c = p.c + (int64_t)row * p.ldc + n0 + col;
      float v = __builtin_ldexpf(sum, unscale);
      if constexpr (ACC) v = *c + v;
      *c = v;
      mx = max(mx, __float_as_uint(v) & 0x7FFFFFFFu);
    }
  }
  if (p.amax) amax_fold(mx, p.amax);
}

// Whether a product takes this kernel: the forward layout (both operands
// contraction-contiguous), exact arithmetic, 3 to 32 output rows, whole
// 256-byte stages, 16-byte aligned rows.
template <bool AK, bool BK>
bool rows_ok(const GemmProblem& p) {
  if constexpr (!(AK && BK)) {
    return false;
  } else {
    if (p.math == kMathNativeFp8 || p.m < kRowsMin || p.m > kRowsMax || p.n < 1) return false;
    if (p.k % kRowsStage != 0) return false;
    auto aligned = [](const void* q, int64_t ld) { return ((uintptr_t)q % 16 == 0) && (ld % 16 == 0); };
    return aligned(p.a, p.lda) && aligned(p.b, p.ldb);
  }
}

template <int MATH, bool ACC>
hipError_t launch_rows_acc(const GemmProblem& p, hipStream_t stream) {
  const dim3 grid((uint32_t)((p.n + 31) / 32)), block(kRowsWaves * 64);
#define FP8LIN_ROWS_CASE(FA, FB)                                                                        \
  if (p.fmt_a == FA && p.fmt_b == FB) {                                                                 \
    hipLaunchKernelGGL((gemm_rows_kernel<FA, FB, MATH, ACC>), grid, block, 0, stream, p);             \
    return hipGetLastError();                                                                           \
  }
  FP8LIN_ROWS_CASE(FP8_E4M3, FP8_E4M3)
  FP8LIN_ROWS_CASE(FP8_E5M2, FP8_E4M3)
  FP8LIN_ROWS_CASE(FP8_E4M3, FP8_E5M2)
  FP8LIN_ROWS_CASE(FP8_E5M2, FP8_E5M2)
#undef FP8LIN_ROWS_CASE
  return hipErrorInvalidValue;
}

template <int MATH>
hipError_t launch_rows(const GemmProblem& p, hipStream_t stream) {
  return p.accumulate ? launch_rows_acc<MATH, true>(p, stream) : launch_rows_acc<MATH, false>(p, stream);
}

}  // namespace gemm_detail
}  // namespace fp8lin
