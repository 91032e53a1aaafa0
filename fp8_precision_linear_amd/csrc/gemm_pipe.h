// Pipelined FP8 product kernel for gfx950: every operand tile streams into LDS
// through LDS DMA (global_load_lds_dwordx4) over a ring of four stages, so
// three contraction stages are always in flight while the MFMAs consume the
// fourth.  No operand byte passes through registers on its way into LDS.
//
// Stage = 64 contraction bytes.  LDS tiles:
//  * contraction-contiguous operand ("K-major", the weight and activation of
//    the forward product, dY in the data gradient): [R rows][64 bytes]; the
//    four 16-byte chunks of row r sit at chunk c ^ ((r >> 1) & 3), so the
//    eight rows a ds_read_b128 quarter-wave touches land in eight different
//    bank groups;
//  * operand whose contraction index is slow in memory ("MN-major": W8 in the
//    data gradient, dY8 and X8 in the weight gradient): the memory tile
//    [64 contraction rows][R bytes] as it is, 16-byte chunk c of row k at
//    c ^ (k & 7).  Fragments are read with ds_read_b64_tr_b8: in each group of
//    16 lanes, lane i receives byte (i & 7) of the 8-byte pieces addressed by
//    lanes 2q + (i >> 3), q = 0..7.  Even lanes address rows kb..kb+7 in the
//    first 8 columns of a 16-column block and odd lanes the same rows in the
//    next 8, so lane i gets the 8 contraction values kb..kb+7 of column i.
//
// Matching the K-major fragment: lane l (row or column l % 32, half h = l / 32)
// holds the stage's contraction bytes [32h, 32h + 32) in ascending order, in
// both layouts.
//
// Ring: four separate __shared__ arrays and a loop unrolled over them, so the
// compiler's LDS-DMA tracking sees that the DMA into one array does not touch
// the array being read; the wait for a stage is an explicit vmcnt that leaves
// the two younger stages in flight, then a bare s_barrier.
#pragma once

#include "gemm_kernel.h"

namespace fp8lin {
namespace gemm_detail {

constexpr int kPipeBK = 64;     // contraction bytes per stage
constexpr int kPipeStages = 4;  // ring depth

typedef int v2i __attribute__((ext_vector_type(2)));

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits [3:0] and
// [15:14], expcnt [6:4] = 7 and lgkmcnt [11:8] = 15 mean "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 3; }

// One LDS-DMA load: 16 bytes per lane from `src` into LDS at
// `lds_kb + 16 * lane` (lds_kb: the wave-uniform LDS byte address of the
// destination KB).  Issued from inline assembly so that the compiler does not
// treat it as a write it must wait for before every later LDS read: the ring
// protocol waits for it explicitly (wait_vmcnt + barrier).  Vector memory
// operations complete in issue order, so the compiler's own vmcnt waits stay
// correct (they can only wait longer).
__device__ __forceinline__ void dma16(const uint8_t* src, const uint8_t* lds_kb) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) const uint8_t*)lds_kb);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory", "m0");
}

// One stage of a K-major tile: rows [row0, row0 + R) x bytes [k0, k0 + 64).
// A wave's DMA fills one KB = 16 rows; lane l lands at byte 16 l, i.e. row
// 16 q + l / 4, physical chunk l % 4, so it fetches logical chunk
// (l % 4) ^ kswz(row).  Rows past the edge re-read the last row (their
// products feed outputs that are not stored).
template <int R>
__device__ __forceinline__ void dma_kmajor(const uint8_t* __restrict__ base, int64_t ld, int row0,
                                           int rows, int k0, uint8_t* lds) {
  const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
#pragma unroll
  for (int b = 0; b < R / 16 / 4; ++b) {
    const int q = wave + 4 * b;
    const int r = q * 16 + (lane >> 2);
    const int gr = min(row0 + r, rows - 1);
    const uint8_t* src = base + (int64_t)gr * ld + k0 + (((lane & 3) ^ kswz(r)) << 4);
    dma16(src, lds + q * 1024);
  }
}

// One stage of an MN-major tile: contraction rows [k0, k0 + 64) x bytes
// [mn0, mn0 + R).  One KB holds 1024 / R rows; lane l lands at row
// q * (1024 / R) + l / (R / 16), physical chunk l % (R / 16), and fetches
// logical chunk (l % (R / 16)) ^ (row & 7).  Chunks past the edge re-read the
// last chunk of the row (mns is a multiple of 16).
template <int R>
__device__ __forceinline__ void dma_mnmajor(const uint8_t* __restrict__ base, int64_t ld, int mn0,
                                            int mns, int k0, uint8_t* lds) {
  constexpr int kChunks = R / 16, kRowsPerKB = 1024 / R;
  const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
#pragma unroll
  for (int b = 0; b < 64 / kRowsPerKB / 4; ++b) {
    const int q = wave + 4 * b;
    const int r = q * kRowsPerKB + lane / kChunks;
    const int c = (lane % kChunks) ^ (r & 7);
    const int gmn = min(mn0 + c * 16, mns - 16);
    const uint8_t* src = base + (int64_t)(k0 + r) * ld + gmn;
    dma16(src, lds + q * 1024);
  }
}

// The lane's 32 contraction bytes of the K-major fragment for tile row r.
__device__ __forceinline__ v8i frag_kmajor(const uint8_t* tile, int r, int h) {
  const uint8_t* row = tile + r * kPipeBK;
  const uint4 x0 = *reinterpret_cast<const uint4*>(row + (((2 * h) ^ kswz(r)) << 4));
  const uint4 x1 = *reinterpret_cast<const uint4*>(row + (((2 * h + 1) ^ kswz(r)) << 4));
  return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

// The lane's 32 contraction bytes of the MN-major fragment for the 32 tile
// columns starting at c0 (lane l takes column c0 + l % 32), via four
// transposing reads of 8 contraction rows each.
template <int R>
__device__ __forceinline__ v8i frag_mnmajor(const uint8_t* tile, int c0, int lane) {
  const int i = lane & 15, h = lane >> 5;
  const int col = c0 + 16 * ((lane >> 4) & 1) + 8 * (i & 1);
  v8i f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 32 * h + 8 * t + (i >> 1);
    const uint8_t* p = tile + row * R + ((((col >> 4) ^ (row & 7))) << 4) + (col & 15);
    const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)p);
    f[2 * t] = v[0];
    f[2 * t + 1] = v[1];
  }
  return f;
}

template <int BM, int BN, bool AK, bool BK, int FA, int FB, int MATH>
struct PipeCtx {
  static constexpr int TM = BM / 64, TN = BN / 64;
  static constexpr int kTileA = BM * kPipeBK;
  // DMA instructions each lane issues per stage (both operands)
  static constexpr int kDmaPerStage = (BM + BN) * kPipeBK / 1024 / 4;

  const GemmProblem& p;
  int m0, n0, nk, lane, wm, wn;
  v16f (&acc)[TM][TN];

  __device__ __forceinline__ void issue(int kt, uint8_t* stage) const {
    const int k0 = kt * kPipeBK;
    if constexpr (AK) dma_kmajor<BM>(p.a, p.lda, m0, p.m, k0, stage);
    else dma_mnmajor<BM>(p.a, p.lda, m0, p.m, k0, stage);
    if constexpr (BK) dma_kmajor<BN>(p.b, p.ldb, n0, p.n, k0, stage + kTileA);
    else dma_mnmajor<BN>(p.b, p.ldb, n0, p.n, k0, stage + kTileA);
  }

  __device__ __forceinline__ void compute(const uint8_t* stage) const {
    const uint8_t* As = stage;
    const uint8_t* Bs = stage + kTileA;
    const int h = lane >> 5, rl = lane & 31;
    v8i af[TM], bf[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (AK) af[i] = frag_kmajor(As, wm * (BM / 2) + i * 32 + rl, h);
      else af[i] = frag_mnmajor<BM>(As, wm * (BM / 2) + i * 32, lane);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (BK) bf[j] = frag_kmajor(Bs, wn * (BN / 2) + j * 32 + rl, h);
      else bf[j] = frag_mnmajor<BN>(Bs, wn * (BN / 2) + j * 32, lane);
    }
    if constexpr (MATH == kMathNativeFp8) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], FA,
                                                                      FB, 0, 127, 0, 127);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v8h ah[TM], bh[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) ah[i] = fp8x8_to_f16<FA>(af[i][2 * q], af[i][2 * q + 1]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bh[j] = fp8x8_to_f16<FB>(bf[j][2 * q], bf[j][2 * q + 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bh[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // Stage kt lives in ring slot S (= kt % 4).  Wait for its DMA (leaving the
  // younger in-flight stages alone), barrier, refill the slot freed by stage
  // kt - 1 with stage kt + 3, then compute stage kt.
  template <int S>
  __device__ __forceinline__ void step(int kt, uint8_t* cur, uint8_t* refill) const {
    if (kt >= nk) return;
    if (kt + 2 < nk) wait_vmcnt<2 * kDmaPerStage>();
    else if (kt + 1 < nk) wait_vmcnt<kDmaPerStage>();
    else wait_vmcnt<0>();
    // A bare barrier: no memory access may move across it (asm "memory"
    // clobber), and it waits for nothing the vmcnt above did not.
    asm volatile("s_barrier" ::: "memory");
    if (kt + 3 < nk) issue(kt + 3, refill);
    compute(cur);
  }
};

template <int BM, int BN, bool AK, bool BK, int FA, int FB, int MATH>
__global__ __launch_bounds__(kThreads) void gemm_pipe_kernel(GemmProblem p, int tiles_m,
                                                             int tiles_n) {
  constexpr int TM = BM / 64, TN = BN / 64;
  constexpr int kStageBytes = (BM + BN) * kPipeBK;
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[kStageBytes];

  int tm, tn;
  tile_coords((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const PipeCtx<BM, BN, AK, BK, FA, FB, MATH> ctx{p, tm * BM, tn * BN, p.k / kPipeBK,
                                                  lane, wave >> 1, wave & 1, acc};
  // prologue: stages 0, 1, 2 in flight
  if (ctx.nk > 0) ctx.issue(0, s0);
  if (ctx.nk > 1) ctx.issue(1, s1);
  if (ctx.nk > 2) ctx.issue(2, s2);
  for (int kt = 0; kt < ctx.nk; kt += kPipeStages) {
    ctx.template step<0>(kt + 0, s0, s3);
    ctx.template step<1>(kt + 1, s1, s0);
    ctx.template step<2>(kt + 2, s2, s1);
    ctx.template step<3>(kt + 3, s3, s2);
  }

  // 32x32 accumulator layout: register r of lane l holds row
  // 8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32 of the MFMA tile.
  const int m0 = tm * BM, n0 = tn * BN, wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, rl = lane & 31;
  const int unscale = -(*p.bias_a + *p.bias_b);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * (BN / 2) + j * 32 + rl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < p.m && col < p.n)
          p.c[(int64_t)row * p.ldc + col] = __builtin_ldexpf(acc[i][j][r], unscale);
      }
    }
}

// ----------------------------------------------------------------- launch

inline dim3 tile_grid(const GemmProblem& p, int bm, int bn, int& tiles_m, int& tiles_n) {
  tiles_m = (p.m + bm - 1) / bm;
  tiles_n = (p.n + bn - 1) / bn;
  return dim3(tiles_m * tiles_n);
}

template <int BM, int BN, bool AK, bool BK, int MATH>
hipError_t launch_pipe(const GemmProblem& p, hipStream_t stream) {
  int tiles_m, tiles_n;
  const dim3 grid = tile_grid(p, BM, BN, tiles_m, tiles_n), block(kThreads);
#define FP8LIN_PIPE_CASE(FA, FB)                                                              \
  if (p.fmt_a == FA && p.fmt_b == FB) {                                                       \
    hipLaunchKernelGGL((gemm_pipe_kernel<BM, BN, AK, BK, FA, FB, MATH>), grid, block, 0,       \
                       stream, p, tiles_m, tiles_n);                                          \
    return hipGetLastError();                                                                 \
  }
  FP8LIN_PIPE_CASE(FP8_E4M3, FP8_E4M3)
  FP8LIN_PIPE_CASE(FP8_E5M2, FP8_E4M3)
  FP8LIN_PIPE_CASE(FP8_E4M3, FP8_E5M2)
  FP8LIN_PIPE_CASE(FP8_E5M2, FP8_E5M2)
#undef FP8LIN_PIPE_CASE
  return hipErrorInvalidValue;
}

template <bool AK, bool BK, int MATH>
hipError_t launch_general(const GemmProblem& p, hipStream_t stream) {
  int tiles_m, tiles_n;
  const dim3 grid = tile_grid(p, 128, 128, tiles_m, tiles_n), block(kThreads);
  const bool vec_a = ((uintptr_t)p.a % 16 == 0) && (p.lda % 16 == 0);
  const bool vec_b = ((uintptr_t)p.b % 16 == 0) && (p.ldb % 16 == 0);
#define FP8LIN_GEN_CASE(FA, FB)                                                               \
  if (p.fmt_a == FA && p.fmt_b == FB) {                                                       \
    hipLaunchKernelGGL((gemm_kernel<128, 128, AK, BK, FA, FB, MATH>), grid, block, 0, stream,  \
                       p, tiles_m, tiles_n, vec_a, vec_b);                                    \
    return hipGetLastError();                                                                 \
  }
  FP8LIN_GEN_CASE(FP8_E4M3, FP8_E4M3)
  FP8LIN_GEN_CASE(FP8_E5M2, FP8_E4M3)
  FP8LIN_GEN_CASE(FP8_E4M3, FP8_E5M2)
  FP8LIN_GEN_CASE(FP8_E5M2, FP8_E5M2)
#undef FP8LIN_GEN_CASE
  return hipErrorInvalidValue;
}

// Fraction of the chip's workgroup slots doing useful work over all waves of
// tiles, weighted by how much of each tile is inside the matrix.
inline double tile_efficiency(int m, int n, int bm, int bn) {
  const int64_t tm = (m + bm - 1) / bm, tn = (n + bn - 1) / bn, tiles = tm * tn;
  const int64_t slots = 256;
  const int64_t waves = (tiles + slots - 1) / slots;
  const double fill = (double)tiles / (double)(waves * slots);
  const double inside = ((double)m * n) / ((double)tm * bm * tn * bn);
  return fill * inside;
}

// FP8LIN_GEMM_TILE=128 or 256 pins the pipelined kernel's tile (tuning and
// tests); otherwise it is chosen from the shape.
inline int forced_tile() {
  const char* s = std::getenv("FP8LIN_GEMM_TILE");
  if (!s) return 0;
  const int v = std::atoi(s);
  return (v == 128 || v == 256) ? v : 0;
}

// The pipelined kernel needs: a contraction that is a whole number of 64-byte
// stages; 16-byte aligned operand rows; and, for an operand read with the
// contraction as its slow index, a row length (M or N) that is a multiple of
// 16.  Anything else runs the general kernel.
template <bool AK, bool BK>
bool pipe_ok(const GemmProblem& p) {
  auto aligned = [](const void* q, int64_t ld) { return ((uintptr_t)q % 16 == 0) && (ld % 16 == 0); };
  if (p.k % kPipeBK != 0) return false;
  if (!aligned(p.a, p.lda) || !aligned(p.b, p.ldb)) return false;
  if (!AK && (p.m % 16 != 0)) return false;
  if (!BK && (p.n % 16 != 0)) return false;
  return true;
}

template <bool AK, bool BK, int MATH>
hipError_t launch_math(const GemmProblem& p, hipStream_t stream) {
  if (!pipe_ok<AK, BK>(p)) return launch_general<AK, BK, MATH>(p, stream);
  // The 256x256 tile does twice the MFMA work per byte of LDS and global
  // traffic of the 128x128 one; prefer it unless it leaves most CUs idle.
  int tile = forced_tile();
  if (tile == 0) {
    const double e256 = tile_efficiency(p.m, p.n, 256, 256);
    const double e128 = tile_efficiency(p.m, p.n, 128, 128) * 0.75;
    tile = e256 >= e128 ? 256 : 128;
  }
  if (tile == 256) return launch_pipe<256, 256, AK, BK, MATH>(p, stream);
  return launch_pipe<128, 128, AK, BK, MATH>(p, stream);
}

template <bool AK, bool BK>
hipError_t launch_layout(const GemmProblem& p, hipStream_t stream) {
  if (p.m <= 0 || p.n <= 0) return hipSuccess;
  if (p.math == kMathNativeFp8) return launch_math<AK, BK, kMathNativeFp8>(p, stream);
  return launch_math<AK, BK, kMathExact>(p, stream);
}

}  // namespace gemm_detail
}  // namespace fp8lin
