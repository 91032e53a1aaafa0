// FP8 x FP8 products with fp32 accumulation for gfx950, unscaled after the
// matmul by 2^-(bias_a + bias_b).
//
// "Training and inference of large language models using 8-bit floating
// point", review page, "Proposed method", bullet 3 (scale before the cast,
// unscale after the matrix multiplication) and bullet 5 (training: forward,
// data-gradient and weight-gradient products; inference).
//
// This file holds what all product kernels share (the arithmetic modes, the
// exact FP8 -> fp16 / bf16 widening, the XCD-aware tile order) and the
// general kernel, which takes any shape and alignment: operands staged
// through registers into two LDS stages of 128 contraction bytes, zero fill
// at every edge, 128x128 tiles of 4 waves.  The pipelined kernels that run
// the workloads' products are in gemm_pipe.h.
//
// Arithmetic:
//  * exact (the default): FP8 codes widened exactly to fp16 or bf16 in
//    registers, then the 32x32x16 fp16 / bf16 MFMA, whose sums keep a 24-bit
//    window (fp32-level accuracy);
//  * native: v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales (E8M0
//    127 = 2^0); the operand formats are instruction fields, so every format
//    pairing runs at the dense FP8 rate, but each instruction keeps only ~13
//    bits below its largest product.
//  * The unscale is one v_ldexp_f32 per output in the epilogue (exact unless
//    the result is an fp32 subnormal).
#pragma once

#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "internal.h"

namespace fp8lin {
namespace gemm_detail {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Product arithmetic.  kMathExact sums products with fp32 accuracy (fp16
// MFMAs on the exactly widened operands); kMathNativeFp8 feeds the FP8 codes
// to the FP8 MFMA, which is twice as fast but sums the 64 products of each
// instruction with only ~13 bits kept below the largest one.
constexpr int kMathExact = FP8LIN_MATH_EXACT;
constexpr int kMathNativeFp8 = FP8LIN_MATH_NATIVE_FP8;
// Exact sums through the bf16 MFMA instead (internal kernel variant; every
// FP8 value is a normal bf16 and bf16 x bf16 products of them are exact).
constexpr int kMathExactBf16 = 100;

constexpr int kThreads = 256;
constexpr int kBK = 128;  // contraction bytes per LDS stage

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 4)) & 7; }

// Byte offset of logical 16-byte chunk c (0..7) of tile row r.
__device__ __forceinline__ int lds_off(int r, int c) { return r * kBK + ((c ^ swz(r)) << 4); }

// Bytes [i, i+16) of a row, zero where i + j >= limit.
__device__ __forceinline__ uint4 load16_partial(const uint8_t* row, int i, int limit) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (i + j < limit) w[j >> 2] |= (uint32_t)row[i + j] << (8 * (j & 3));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

__device__ __forceinline__ uint32_t byte_of(const uint4& v, int j) {
  return (word_of(v, j >> 2) >> (8 * (j & 3))) & 0xFFu;
}

// Loader interface: load(...) fetches one stage of the operand tile into
// registers; store(lds) writes it into the LDS tile.  The stage is complete
// in LDS once every lane has passed store() and a barrier.

// Operand tile whose contraction index is contiguous in memory:
// rows [row0, row0 + R) x bytes [k0, k0 + 128), through registers, with
// zero fill past the edges (any contraction length).
template <int R>
struct KMajorLoader {
  static constexpr int kChunks = R * (kBK / 16) / kThreads;  // 16-byte chunks per lane
  uint4 v[kChunks];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ base, int64_t ld, int row0,
                                       int rows, int k0, int K, bool vec, uint8_t*) {
#pragma unroll
    for (int p = 0; p < kChunks; ++p) {
      const int q = (int)threadIdx.x + kThreads * p, r = q >> 3, c = q & 7;
      const int gr = row0 + r, gk = k0 + c * 16;
      if (gr < rows && gk < K) {
        const uint8_t* src = base + (int64_t)gr * ld;
        if (vec && gk + 16 <= K)
          v[p] = *reinterpret_cast<const uint4*>(src + gk);
        else
          v[p] = load16_partial(src, gk, K);
      } else {
        v[p] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
    for (int p = 0; p < kChunks; ++p) {
      const int q = (int)threadIdx.x + kThreads * p, r = q >> 3, c = q & 7;
      *reinterpret_cast<uint4*>(lds + lds_off(r, c)) = v[p];
    }
  }
};

// Operand tile whose contraction index is the slow one in memory: memory rows
// [k0, k0 + 128) x bytes [mn0, mn0 + R).  Each lane loads KU memory rows of 16
// bytes and writes 16 tile rows of KU contraction bytes.
template <int R>
struct MNMajorLoader {
  static constexpr int KU = R / 32;  // contraction rows per lane (8 or 4)
  static constexpr int NU = R / 16;  // 16-byte column groups across the tile
  static_assert(KU == 8 || KU == 4, "tile size");
  uint4 v[KU];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ base, int64_t ld, int mn0,
                                       int mns, int k0, int K, bool vec, uint8_t*) {
    const int mu = (int)threadIdx.x % NU, kb = (int)threadIdx.x / NU;
    const int gmn = mn0 + mu * 16;
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int gk = k0 + kb * KU + i;
      if (gk < K && gmn < mns) {
        const uint8_t* src = base + (int64_t)gk * ld;
        if (vec && gmn + 16 <= mns)
          v[i] = *reinterpret_cast<const uint4*>(src + gmn);
        else
          v[i] = load16_partial(src, gmn, mns);
      } else {
        v[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int mu = (int)threadIdx.x % NU, kb = (int)threadIdx.x / NU;
    const int kbyte = kb * KU;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = mu * 16 + j;
      uint8_t* dst = lds + r * kBK + (((kbyte >> 4) ^ swz(r)) << 4) + (kbyte & 15);
      const uint32_t lo = byte_of(v[0], j) | (byte_of(v[1], j) << 8) | (byte_of(v[2], j) << 16) |
                          (byte_of(v[3], j) << 24);
      if constexpr (KU == 8) {
        const uint32_t hi = byte_of(v[4], j) | (byte_of(v[5], j) << 8) |
                            (byte_of(v[6], j) << 16) | (byte_of(v[7], j) << 24);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<uint32_t*>(dst) = lo;
      }
    }
  }
};

// Block bid's output tile.  Workgroup bid runs on XCD bid % 8: when the tile
// count allows, each XCD takes a contiguous run of the tile order, so the
// tiles it runs at once share operand panels in its L2.  The order walks
// groups of G tile-rows column by column.  With G = 4 a 32-tile-row output
// (8192 rows) gives each XCD one group of 4 rows across every column, and the
// eight XCDs walk the columns (the weight panels) together: 1.1-1.3% faster
// on the Llama-2-70B products than G = 8 (two runs each; G = 2 the same as
// 4, G = 16 half the gain, G = 32 none; the 13B gradients within noise).
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int t = bid;
  if ((total & 7) == 0) t = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int G = 4;
  const int width = G * tiles_n;
  const int first_m = (t / width) * G;
  const int gsize = min(tiles_m - first_m, G);
  tm = first_m + (t % width) % gsize;
  tn = (t % width) / gsize;
}

// Four FP8 codes (one dword) as four fp16 values (two dwords), exactly.
// E5M2 shares fp16's sign, exponent width and bias: its code is the high byte
// of the fp16 with the same value (subnormals, inf and NaN included).  Every
// E4M3 value is a normal fp16; v_cvt_scalef32_pk_f16_fp8 with scale 1 converts
// two codes (the low or the high 16-bit word of the dword) per instruction,
// exactly for every finite code and NaN to NaN (measured over all 65536 code
// pairs, both words).  Its result is taken as one 32-bit pattern: extracting
// the two halves separately has been compiled into a repeat of the low half.
template <int FMT>
__device__ __forceinline__ uint2 fp8x4_to_f16(uint32_t w) {
  if constexpr (FMT == FP8_E5M2) {
    // one v_perm_b32 per output dword: bytes (high to low) [c1, 0, c0, 0] and
    // [c3, 0, c2, 0] of the dword's codes c0..c3 (selector 0x0C reads a zero byte)
    return make_uint2(__builtin_amdgcn_perm(0u, w, 0x010C000Cu), __builtin_amdgcn_perm(0u, w, 0x030C020Cu));
  } else {
    return make_uint2(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)));
  }
}

// Four FP8 codes as four bf16 values (two dwords), exactly: every E4M3 and
// E5M2 value is a normal bf16.  One v_cvt_scalef32_pk_bf16_{fp8,bf8} (scale 1)
// per two codes; the result is read as one 32-bit pattern.
template <int FMT>
__device__ __forceinline__ uint2 fp8x4_to_bf16(uint32_t w) {
  if constexpr (FMT == FP8_E5M2) {
    return make_uint2(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true)));
  } else {
    return make_uint2(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
  }
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int FMT>
__device__ __forceinline__ v8bf fp8x8_to_bf16(int w0, int w1) {
  const uint2 a = fp8x4_to_bf16<FMT>((uint32_t)w0), b = fp8x4_to_bf16<FMT>((uint32_t)w1);
  return __builtin_bit_cast(v8bf, make_uint4(a.x, a.y, b.x, b.y));
}

template <int FMT>
__device__ __forceinline__ v8h fp8x8_to_f16(int w0, int w1) {
  const uint2 a = fp8x4_to_f16<FMT>((uint32_t)w0), b = fp8x4_to_f16<FMT>((uint32_t)w1);
  return __builtin_bit_cast(v8h, make_uint4(a.x, a.y, b.x, b.y));
}

// Fold this lane's largest output magnitude (fp32 bits, sign cleared) into
// *amax: wave maximum by shuffles, then one atomicMax per wave -- skipped when
// *amax already holds at least as much.  Every wave of a product reaches this
// at about the same time, and atomics on one address serialise; the value only
// grows, so a stale read can cost an unneeded atomic but never a wrong result.
// Every lane of the wave must reach it.
__device__ __forceinline__ void amax_fold(uint32_t m, uint32_t* amax) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0 &&
      m > __hip_atomic_load(amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    atomicMax(amax, m);
}

// The general kernel: any shape and alignment (operands staged through
// registers with zero fill at every edge, two LDS stages of 128 bytes).
template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, int FA, int FB, int MATH>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmProblem p, int tiles_m, int tiles_n,
                                                        bool vec_a, bool vec_b) {
  constexpr int TM = BM / 64, TN = BN / 64;  // 32x32 MFMA tiles per wave
  constexpr int kStage = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  using LoaderA = typename std::conditional<A_KMAJOR, KMajorLoader<BM>, MNMajorLoader<BM>>::type;
  using LoaderB = typename std::conditional<B_KMAJOR, KMajorLoader<BN>, MNMajorLoader<BN>>::type;

  int tm, tn;
  tile_coords((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  LoaderA la;
  LoaderB lb;
  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (p.k + kBK - 1) / kBK;
  if (nk > 0) {
    la.load(p.a, p.lda, m0, p.m, 0, p.k, vec_a, smem);
    lb.load(p.b, p.ldb, n0, p.n, 0, p.k, vec_b, smem + BM * kBK);
    la.store(smem);
    lb.store(smem + BM * kBK);
    __syncthreads();
  }

  const int h = lane >> 5, rl = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* cur = smem + (kt & 1) * kStage;
    uint8_t* nxt = smem + ((kt + 1) & 1) * kStage;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(p.a, p.lda, m0, p.m, (kt + 1) * kBK, p.k, vec_a, nxt);
      lb.load(p.b, p.ldb, n0, p.n, (kt + 1) * kBK, p.k, vec_b, nxt + BM * kBK);
    }
    const uint8_t* As = cur;
    const uint8_t* Bs = cur + BM * kBK;
#pragma unroll
    for (int s = 0; s < kBK / 64; ++s) {
      const int c0 = s * 4 + h * 2;  // this lane's 32 contraction bytes: chunks c0, c0 + 1
      v8i af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * (BM / 2) + i * 32 + rl;
        const uint4 x0 = *reinterpret_cast<const uint4*>(As + lds_off(r, c0));
        const uint4 x1 = *reinterpret_cast<const uint4*>(As + lds_off(r, c0 + 1));
        af[i] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                    (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * (BN / 2) + j * 32 + rl;
        const uint4 x0 = *reinterpret_cast<const uint4*>(Bs + lds_off(r, c0));
        const uint4 x1 = *reinterpret_cast<const uint4*>(Bs + lds_off(r, c0 + 1));
        bf[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                    (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
      if constexpr (MATH == kMathNativeFp8) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bf[j], acc[i][j], FA, FB, 0, 127, 0, 127);
      } else {
        // Exact math: the lane's 32 codes become 32 fp16 values (no rounding:
        // every E4M3 and E5M2 value is an fp16 value) fed to four 32x32x16
        // fp16 MFMAs; step q takes the lane's bytes [8q, 8q + 8), the same
        // contraction indices in A and B.
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
    if (more) {
      la.store(nxt);
      lb.store(nxt + BM * kBK);
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: register r of lane l holds row
  // 8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32 of the MFMA tile.
  // With p.accumulate the 16 outputs of a tile are read (all issued) before
  // the unscaled sums are added to them and stored.
  const int unscale = -(*p.bias_a + *p.bias_b);
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * (BN / 2) + j * 32 + rl;
      float old[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        old[r] = (p.accumulate && row < p.m && col < p.n) ? p.c[(int64_t)row * p.ldc + col] : 0.0f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < p.m && col < p.n) {
          float v = __builtin_ldexpf(acc[i][j][r], unscale);
          if (p.accumulate) v = old[r] + v;
          p.c[(int64_t)row * p.ldc + col] = v;
          mx = max(mx, __float_as_uint(v) & 0x7FFFFFFFu);
        }
      }
    }
  if (p.amax) amax_fold(mx, p.amax);
}

}  // namespace gemm_detail
}  // namespace fp8lin
