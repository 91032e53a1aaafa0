// Pipelined FP8 product kernels for gfx950: every operand tile streams into
// LDS through LDS DMA (global_load_lds_dwordx4) over a ring of four stages, so
// three contraction stages are in flight while the MFMAs consume the fourth.
// No operand byte passes through registers on its way into LDS.
//
// Stage = 64 contraction bytes.  LDS tiles:
//  * contraction-contiguous operand ("K-major", the weight and activation of
//    the forward product, dY in the data gradient): [R rows][64 bytes]; the
//    four 16-byte chunks of row r sit at chunk c ^ ((r >> 2) & 3).  The LDS
//    has 64 banks (256 bytes per cycle): the 16 rows that 16 lanes of a
//    ds_read_b128 address (four rows per 256-byte bank window) then cover all
//    16 bank groups of 16 bytes;
//  * operand whose contraction index is slow in memory ("MN-major": W8 in the
//    data gradient, dY8 and X8 in the weight gradient): the memory tile
//    [64 contraction rows][R bytes] as it is, 16-byte chunk c of row k at
//    c ^ mnswz(k) (mnswz: (k & 7) for 128-byte rows, 2 (k & 7) for 256-byte
//    rows; either way the 8 rows x 2 column blocks that 32 lanes of one
//    transposing read address fall in 16 different bank groups).
//    Fragments are read with ds_read_b64_tr_b8: in each group of
//    16 lanes, lane i receives byte (i & 7) of the 8-byte pieces addressed by
//    lanes 2q + (i >> 3), q = 0..7.  Even lanes address rows kb..kb+7 in the
//    first 8 columns of a 16-column block and odd lanes the same rows in the
//    next 8, so lane i gets the 8 contraction values kb..kb+7 of column i.
//
// Matching the K-major fragment: lane l (row or column l % 32, half h = l / 32)
// holds the stage's contraction bytes [32h, 32h + 32) in ascending order, in
// both layouts.
//
// Two kernels share these pieces:
//  * gemm_pp_kernel, 256x256 tiles, 8 waves in two groups of four ("ping-
//    pong").  Each SIMD holds one wave of each group.  The groups are half a
//    stage apart: while one group issues its MFMAs from fragments already in
//    registers, the other reads the next stage's fragments from LDS and
//    issues DMA, and a barrier swaps the roles.  A wave's MFMA phase is never
//    interrupted by LDS latency, and the matrix core of each SIMD alternates
//    between the two waves.  Group 0 computes tile rows [0, 128) and streams
//    the A tile, group 1 rows [128, 256) and the B tile; wave w of a group
//    computes 64 tile columns.
//  * gemm_quad_kernel, 128x128 tiles, 4 waves (2 x 2) that read and multiply
//    in the same phase; used where 256x256 tiles would leave CUs idle.
//
// Ring: one __shared__ array per operand holding its four stage tiles, and
// main loops unrolled over the four slots, so every slot and fragment offset
// is an instruction constant on top of a few per-lane base registers.  The
// wait for a stage is an explicit vmcnt that leaves the two younger stages of
// the wave's own DMA in flight, then a bare s_barrier.
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

// s_waitcnt lgkmcnt(0) only: every LDS read this wave issued has returned.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Wait until at most `younger` stages of this wave's DMA (D instructions per
// stage) are still in flight.
template <int D>
__device__ __forceinline__ void wait_stages(int younger) {
  if (younger >= 2) wait_vmcnt<2 * D>();
  else if (younger == 1) wait_vmcnt<D>();
  else wait_vmcnt<0>();
}

// A bare barrier: no memory access may move across it (asm "memory" clobber),
// and it waits for nothing the explicit waits did not.
__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Chunk swizzles of the K-major and MN-major stage tiles.
__device__ __forceinline__ int kswz(int r) { return (r >> 2) & 3; }
template <int R>
__device__ __forceinline__ int mnswz(int k) { return R == 256 ? 2 * (k & 7) : (k & 7); }

// The wave's index in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
}

// Opaque copies: the value is the same, but the compiler cannot hoist address
// arithmetic built on it out of the main loop.  Without them it precomputes a
// separate register for every (ring slot, fragment) address and spills.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ int64_t opaque64(int64_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// One LDS-DMA load: 16 bytes per lane from `src` into LDS at
// `lds_kb + 16 * lane` (lds_kb: the wave-uniform LDS byte address of the
// destination KB).  Issued from inline assembly so that the compiler does not
// treat it as a write it must wait for before every later LDS read: the ring
// protocol waits for it explicitly (wait_vmcnt + barrier).  Vector memory
// operations complete in issue order, so the compiler's own vmcnt waits stay
// correct (they can only wait longer).
__device__ __forceinline__ void dma16(const uint8_t* src, uint32_t lds_kb) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_kb))
      : "memory", "m0");
}

// The DMA loads one wave issues per stage for an R-wide operand tile, shared
// among NW waves (w = this wave's index among them).  One load fills one KB
// of the stage tile: KB q = w + NW * b.
//  * K-major, tile rows [mn0, mn0 + R) x bytes [k0, k0 + 64): KB q holds
//    rows 16 q .. 16 q + 15; lane l lands at byte 16 l, i.e. row 16 q + l / 4,
//    physical chunk l % 4, so it fetches logical chunk (l % 4) ^ kswz(row).
//    Rows past the edge re-read the last row (their products feed outputs
//    that are not stored).
//  * MN-major, contraction rows [k0, k0 + 64) x bytes [mn0, mn0 + R): KB q
//    holds 1024 / R rows; lane l lands at row q * (1024 / R) + l / (R / 16),
//    physical chunk l % (R / 16), and fetches logical chunk
//    (l % (R / 16)) ^ mnswz(row).  Chunks past the edge re-read the last chunk
//    of the row (mns is a multiple of 16).
// off[b] is the lane's byte offset from the operand base for stage 0; stage
// kt adds kt * 64 (K-major) or kt * 64 * ld (MN-major).
template <int R, bool KMAJ, int NW>
struct DmaPlan {
  static constexpr int kRowsPerKB = KMAJ ? 16 : 1024 / R;
  static constexpr int N = R * kPipeBK / 1024 / NW;  // the stage tile's KBs over NW waves
  static_assert(N >= 1 && N * NW * 1024 == R * kPipeBK, "KB split");
  int64_t off[N];
  int w;

  __device__ __forceinline__ void init(int64_t ld, int mn0, int mns, int wave, int lane) {
    w = wave;
#pragma unroll
    for (int b = 0; b < N; ++b) {
      const int q = w + NW * b;
      if constexpr (KMAJ) {
        const int r = q * 16 + (lane >> 2);
        const int gr = min(mn0 + r, mns - 1);
        off[b] = (int64_t)gr * ld + (((lane & 3) ^ kswz(r)) << 4);
      } else {
        constexpr int kChunks = R / 16;
        const int r = q * kRowsPerKB + lane / kChunks;
        const int c = (lane % kChunks) ^ mnswz<R>(r);
        const int gmn = min(mn0 + c * 16, mns - 16);
        off[b] = (int64_t)r * ld + gmn;
      }
    }
  }

  // Stage kt into the stage tile at LDS address `lds_tile`.
  __device__ __forceinline__ void issue(const uint8_t* base, int64_t ld, int kt,
                                        uint32_t lds_tile) const {
    const int64_t kofs = KMAJ ? (int64_t)kt * kPipeBK : (int64_t)kt * kPipeBK * ld;
#pragma unroll
    for (int b = 0; b < N; ++b) dma16(base + kofs + opaque64(off[b]), lds_tile + (w + NW * b) * 1024);
  }
};

// Where a wave's T fragments of an R-wide operand tile sit in LDS: the
// fragment of the 32 rows (K-major) or columns (MN-major) first + 32 t.
//  * K-major: lane l (row r = first + 32 t + l % 32, half h = l / 32) reads
//    logical chunks 2h and 2h + 1 of row r with two ds_read_b128.  first is a
//    multiple of 16, so the swizzle depends on l % 32 alone and the offsets of
//    fragment t differ by the constant 32 t * 64.
//  * MN-major: four ds_read_b64_tr_b8 of 8 contraction rows each (rows
//    32h + 8u + (l % 16) / 2, u = 0..3, at a constant distance 8 R apart); even
//    lanes address the first 8 columns of a 16-column block and odd lanes the
//    next 8, so lane l receives the 8 contraction values of column
//    first + 32 t + l % 32.
// off[] holds the lane's LDS byte addresses in ring slot 0 (slot s adds the
// constant s * R * 64).
template <int R, bool KMAJ, int T>
struct FragPlan {
  static constexpr int N = KMAJ ? 2 : T;
  uint32_t off[N];

  __device__ __forceinline__ void init(uint32_t tile0, int first, int lane) {
    const int h = lane >> 5;
    if constexpr (KMAJ) {
      const int rl = lane & 31;
      off[0] = tile0 + (first + rl) * kPipeBK + (((2 * h) ^ kswz(rl)) << 4);
      off[1] = tile0 + (first + rl) * kPipeBK + (((2 * h + 1) ^ kswz(rl)) << 4);
    } else {
      const int i = lane & 15, lb = (lane >> 4) & 1;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int blk = ((first + 32 * t) >> 4) + lb;  // 16-byte column block
        off[t] = tile0 + (32 * h + (i >> 1)) * R + ((blk ^ mnswz<R>(i >> 1)) << 4) + 8 * (i & 1);
      }
    }
  }

  template <int SLOT>
  __device__ __forceinline__ v8i load(int t) const {
    return load_at(SLOT * R * kPipeBK, t);
  }

  // Fragment t of the ring slot that starts kSlot bytes after slot 0.
  __device__ __forceinline__ v8i load_at(uint32_t kSlot, int t) const {
    typedef int v4i __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const v4i* lds_v4i;
    typedef __attribute__((address_space(3))) v2i* lds_v2i;
    if constexpr (KMAJ) {
      const uint32_t kt = kSlot + t * 32 * kPipeBK;
      const v4i x0 = *(lds_v4i)(uintptr_t)(opaque(off[0]) + kt);
      const v4i x1 = *(lds_v4i)(uintptr_t)(opaque(off[1]) + kt);
      return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    } else {
      const uint32_t a = opaque(off[t]) + kSlot;
      v8i f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(uintptr_t)(a + 8 * u * R));
        f[2 * u] = v[0];
        f[2 * u + 1] = v[1];
      }
      return f;
    }
  }
};

// Register fences: empty volatile asm that claims to rewrite the values.
// Volatile asm keeps its order against the barrier asm, so an MFMA phase whose
// inputs are fenced at its start and outputs at its end stays between the
// barriers that delimit it (plain register arithmetic may otherwise be moved
// across an s_barrier written as inline asm).
template <int N>
__device__ __forceinline__ void fence(v8i (&f)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(f[i]));
}
template <int TM, int TN>
__device__ __forceinline__ void fence(v16f (&acc)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(acc[i][j]));
}

// acc[i][j] += A-fragment i x B-fragment j over one 64-byte stage.
template <int TM, int TN, int FA, int FB, int MATH>
__device__ __forceinline__ void mma_stage(const v8i (&af)[TM], const v8i (&bf)[TN],
                                          v16f (&acc)[TM][TN]) {
  if constexpr (MATH == kMathNativeFp8) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], FA, FB,
                                                                    0, 127, 0, 127);
  } else if constexpr (MATH == kMathExactBf16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v8bf ah[TM], bh[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) ah[i] = fp8x8_to_bf16<FA>(af[i][2 * q], af[i][2 * q + 1]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bh[j] = fp8x8_to_bf16<FB>(bf[j][2 * q], bf[j][2 * q + 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
    }
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

template <int TM, int TN>
__device__ __forceinline__ void zero_acc(v16f (&acc)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// Unscale and store a wave's TM x TN block of 32x32 tiles whose top-left
// output is (row0, col0).  32x32 accumulator layout: register r of lane l
// holds row 8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32.  With
// AMAX the largest stored magnitude is folded into *p.amax.  The stores are
// non-temporal: the output is not read back by the product, and a wave of
// tiles writes about twice an XCD's L2 in outputs (measured: 0.2-1% faster).
template <bool AMAX, int TM, int TN>
__device__ __forceinline__ void store_block_as(const GemmProblem& p, const v16f (&acc)[TM][TN],
                                               int row0, int col0, int lane) {
  const int h = lane >> 5, rl = lane & 31;
  const int unscale = -(*p.bias_a + *p.bias_b);
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = col0 + j * 32 + rl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < p.m && col < p.n) {
          const float v = __builtin_ldexpf(acc[i][j][r], unscale);
          __builtin_nontemporal_store(v, &p.c[(int64_t)row * p.ldc + col]);
          if constexpr (AMAX) mx = max(mx, __float_as_uint(v) & 0x7FFFFFFFu);
        }
      }
    }
  if constexpr (AMAX) amax_fold(mx, p.amax);
}

// The same block added into the output: out = old + the unscaled sum, one
// fp32 addition per element.  The old values of tile-row i + 1 are loaded
// before tile-row i is added and stored (two rows of them in registers), so
// only the first row's read latency is exposed.  Addresses are one per-lane
// pointer (row0 + 4h, col0 + lane % 32) plus a row offset that is the same
// for every lane, which keeps the 64-bit address arithmetic out of the
// vector registers that hold the old values.
template <int TM, int TN>
__device__ __forceinline__ void accumulate_block(const GemmProblem& p, const v16f (&acc)[TM][TN],
                                                 int row0, int col0, int lane) {
  const int h = lane >> 5, rl = lane & 31;
  const int unscale = -(*p.bias_a + *p.bias_b);
  const int rlane = row0 + 4 * h, clane = col0 + rl;
  float* const q = p.c + (int64_t)rlane * p.ldc + clane;
  // element (i, j, r): row rlane + dr, column clane + 32 j, dr = 32 i + 8 (r / 4) + r % 4
  auto in = [&](int dr, int j) { return rlane + dr < p.m && clane + 32 * j < p.n; };
  auto at = [&](int dr, int j) { return q + (int64_t)dr * p.ldc + 32 * j; };
  float old[2][TN][16];
  auto load_row = [&](int i, float (&o)[TN][16]) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dr = 32 * i + 8 * (r >> 2) + (r & 3);
        o[j][r] = in(dr, j) ? *at(dr, j) : 0.0f;
      }
  };
  load_row(0, old[0]);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i + 1 < TM) load_row(i + 1, old[(i + 1) & 1]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dr = 32 * i + 8 * (r >> 2) + (r & 3);
        if (in(dr, j))
          __builtin_nontemporal_store(old[i & 1][j][r] + __builtin_ldexpf(acc[i][j][r], unscale), at(dr, j));
      }
  }
}

// The epilogue of a kernel instantiated with ACC (fp8_scaled_gemm_accumulate,
// which never asks for the output's amax) or without it (the amax optional).
// The accumulating epilogue is its own instantiation so that the common one
// keeps its code and registers (a runtime choice between the two in one
// kernel cost the 70B QKV product ~2%).
template <bool ACC, int TM, int TN>
__device__ __forceinline__ void store_block(const GemmProblem& p, const v16f (&acc)[TM][TN],
                                            int row0, int col0, int lane) {
  if constexpr (ACC) accumulate_block(p, acc, row0, col0, lane);
  else if (p.amax) store_block_as<true>(p, acc, row0, col0, lane);
  else store_block_as<false>(p, acc, row0, col0, lane);
}

// ------------------------------------------------------ ping-pong, 256 x 256

// The work of one wave of group G (0 or 1) in the ping-pong kernel.
//  * Fragments: A rows G * 128 + 32 i (i < 4), B columns 64 gw + 32 j (j < 2).
//  * DMA: group 0 streams the A tile, group 1 the B tile, 16 KB per stage
//    each, four loads per wave.
//  * Stage kt: phase 2kt, group 0 reads stage kt while group 1 multiplies
//    stage kt - 1; phase 2kt + 1, group 0 multiplies stage kt while group 1
//    reads it.  A barrier separates the phases.  Before the first of them
//    every wave waits for its own DMA of stage kt (the two younger stages stay
//    in flight), so after it the whole stage is in LDS.  The refill of the
//    slot stage kt - 1 used (with stage kt + 3) is issued in the read phase:
//    both groups finished reading stage kt - 1 before phase 2kt.  A read
//    phase ends with the wave's fragments in registers, so a slot is never
//    overwritten while a read of it is outstanding.
template <int G, bool AK, bool BK, int FA, int FB, int MATH>
struct PingPongWave {
  static constexpr int R = 256, TM = 4, TN = 2;
  static constexpr bool SK = G == 0 ? AK : BK;  // layout of the streamed operand
  using Dma = DmaPlan<R, SK, 4>;

  const GemmProblem& p;
  int nk;
  uint32_t lds_mine;  // LDS address of slot 0 of the streamed operand's tile
  const uint8_t* base;
  int64_t ld;
  Dma dma;
  FragPlan<R, AK, TM> fa;
  FragPlan<R, BK, TN> fb;
  v8i af[TM], bf[TN];
  v16f (&acc)[TM][TN];

  __device__ __forceinline__ PingPongWave(const GemmProblem& p_, int m0, int n0, int gw, int lane,
                                          uint32_t lds_a, uint32_t lds_b, v16f (&acc_)[TM][TN])
      : p(p_), nk(p_.k / kPipeBK), acc(acc_) {
    lds_mine = G == 0 ? lds_a : lds_b;
    base = G == 0 ? p.a : p.b;
    ld = G == 0 ? p.lda : p.ldb;
    dma.init(ld, G == 0 ? m0 : n0, G == 0 ? p.m : p.n, gw, lane);
    fa.init(lds_a, G * (R / 2), lane);
    fb.init(lds_b, gw * (R / 4), lane);
  }

  template <int SLOT>
  __device__ __forceinline__ void read(int kt) {
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = fa.template load<SLOT>(i);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = fb.template load<SLOT>(j);
    if (kt + 3 < nk) dma.issue(base, ld, kt + 3, lds_mine + ((SLOT + 3) % 4) * R * kPipeBK);
    wait_lgkm0();
  }

  __device__ __forceinline__ void mma() {
    fence(af);
    fence(bf);
    mma_stage<TM, TN, FA, FB, MATH>(af, bf, acc);
    fence(acc);
  }

  template <int SLOT>
  __device__ __forceinline__ void step(int kt) {
    if (kt >= nk) return;
    wait_stages<Dma::N>(min(2, nk - 1 - kt));
    bare_barrier();
    if constexpr (G == 0) read<SLOT>(kt);
    else if (kt > 0) mma();
    bare_barrier();
    if constexpr (G == 0) mma();
    else read<SLOT>(kt);
  }

  __device__ __forceinline__ void run() {
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < nk) dma.issue(base, ld, s, lds_mine + s * R * kPipeBK);
    for (int kt = 0; kt < nk; kt += kPipeStages) {
      step<0>(kt + 0);
      step<1>(kt + 1);
      step<2>(kt + 2);
      step<3>(kt + 3);
    }
    if (G == 1 && nk > 0) mma();  // group 1's last stage
  }
};

template <bool AK, bool BK, int FA, int FB, int MATH, bool ACC>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmProblem p, int tiles_m, int tiles_n) {
  constexpr int R = 256;
  // Ring of four stages per operand: slot s of A at sa + s * 16 KB, of B at
  // sb + s * 16 KB (all fragment offsets stay below 64 KB of their base).
  __shared__ __attribute__((aligned(1024))) uint8_t sa[kPipeStages * R * kPipeBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sb[kPipeStages * R * kPipeBK];

  int tm, tn;
  tile_coords((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int lane = (int)threadIdx.x & 63, wave = wave_id();
  const int g = wave >> 2, gw = wave & 3;
  const int m0 = tm * R, n0 = tn * R;

  v16f acc[4][2];
  zero_acc(acc);
  if (g == 0) {
    PingPongWave<0, AK, BK, FA, FB, MATH> w(p, m0, n0, gw, lane, lds_addr(sa), lds_addr(sb), acc);
    w.run();
  } else {
    PingPongWave<1, AK, BK, FA, FB, MATH> w(p, m0, n0, gw, lane, lds_addr(sa), lds_addr(sb), acc);
    w.run();
  }
  store_block<ACC>(p, acc, m0 + g * (R / 2), n0 + gw * (R / 4), lane);
}

// ---------------------------------------------------------- quad, 128 x 128

// 4 waves in a 2 x 2 grid; wave (wm, wn) owns a 64 x 64 block and issues a
// quarter of both operand tiles' DMA.  Each stage: wait for it, barrier,
// refill the slot freed by stage kt - 1 with stage kt + 3, read, multiply.
template <bool AK, bool BK, int FA, int FB, int MATH>
struct QuadWave {
  static constexpr int R = 128, TM = 2, TN = 2;
  using DmaA = DmaPlan<R, AK, 4>;
  using DmaB = DmaPlan<R, BK, 4>;

  const GemmProblem& p;
  int nk;
  uint32_t lds_a, lds_b;
  DmaA da;
  DmaB db;
  FragPlan<R, AK, TM> fa;
  FragPlan<R, BK, TN> fb;
  v16f (&acc)[TM][TN];

  __device__ __forceinline__ QuadWave(const GemmProblem& p_, int m0, int n0, int wave, int lane,
                                      uint32_t la, uint32_t lb, v16f (&acc_)[TM][TN])
      : p(p_), nk(p_.k / kPipeBK), lds_a(la), lds_b(lb), acc(acc_) {
    da.init(p.lda, m0, p.m, wave, lane);
    db.init(p.ldb, n0, p.n, wave, lane);
    fa.init(la, (wave >> 1) * (R / 2), lane);
    fb.init(lb, (wave & 1) * (R / 2), lane);
  }

  __device__ __forceinline__ void issue(int kt, int slot) const {
    da.issue(p.a, p.lda, kt, lds_a + slot * R * kPipeBK);
    db.issue(p.b, p.ldb, kt, lds_b + slot * R * kPipeBK);
  }

  template <int SLOT>
  __device__ __forceinline__ void step(int kt) {
    if (kt >= nk) return;
    wait_stages<DmaA::N + DmaB::N>(min(2, nk - 1 - kt));
    bare_barrier();
    if (kt + 3 < nk) issue(kt + 3, (SLOT + 3) % 4);
    v8i af[TM], bf[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = fa.template load<SLOT>(i);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = fb.template load<SLOT>(j);
    mma_stage<TM, TN, FA, FB, MATH>(af, bf, acc);
  }

  __device__ __forceinline__ void run() {
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < nk) issue(s, s);
    for (int kt = 0; kt < nk; kt += kPipeStages) {
      step<0>(kt + 0);
      step<1>(kt + 1);
      step<2>(kt + 2);
      step<3>(kt + 3);
    }
  }
};

template <bool AK, bool BK, int FA, int FB, int MATH, bool ACC>
__global__ __launch_bounds__(256) void gemm_quad_kernel(GemmProblem p, int tiles_m, int tiles_n) {
  constexpr int R = 128;
  __shared__ __attribute__((aligned(1024))) uint8_t sa[kPipeStages * R * kPipeBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sb[kPipeStages * R * kPipeBK];

  int tm, tn;
  tile_coords((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int lane = (int)threadIdx.x & 63, wave = wave_id();
  const int m0 = tm * R, n0 = tn * R;

  v16f acc[2][2];
  zero_acc(acc);
  QuadWave<AK, BK, FA, FB, MATH> w(p, m0, n0, wave, lane, lds_addr(sa), lds_addr(sb), acc);
  w.run();
  store_block<ACC>(p, acc, m0 + (wave >> 1) * (R / 2), n0 + (wave & 1) * (R / 2), lane);
}

}  // namespace gemm_detail
}  // namespace fp8lin

#include "gemm_gemv.h"
#include "gemm_rows.h"

namespace fp8lin {
namespace gemm_detail {

// ----------------------------------------------------------------- launch

inline dim3 tile_grid(const GemmProblem& p, int bm, int bn, int& tiles_m, int& tiles_n) {
  tiles_m = (p.m + bm - 1) / bm;
  tiles_n = (p.n + bn - 1) / bn;
  return dim3(tiles_m * tiles_n);
}

// Instantiate KERNEL<AK, BK, FA, FB, MATH, ACC> for the operand formats of p.
#define FP8LIN_FORMAT_DISPATCH(KERNEL, GRID, BLOCK, ACC)                                           \
  do {                                                                                             \
    if (p.fmt_a == FP8_E4M3 && p.fmt_b == FP8_E4M3) {                                              \
      hipLaunchKernelGGL((KERNEL<AK, BK, FP8_E4M3, FP8_E4M3, MATH, ACC>), GRID, BLOCK, 0, stream,  \
                         p, tiles_m, tiles_n);                                                     \
    } else if (p.fmt_a == FP8_E5M2 && p.fmt_b == FP8_E4M3) {                                       \
      hipLaunchKernelGGL((KERNEL<AK, BK, FP8_E5M2, FP8_E4M3, MATH, ACC>), GRID, BLOCK, 0, stream,  \
                         p, tiles_m, tiles_n);                                                     \
    } else if (p.fmt_a == FP8_E4M3 && p.fmt_b == FP8_E5M2) {                                       \
      hipLaunchKernelGGL((KERNEL<AK, BK, FP8_E4M3, FP8_E5M2, MATH, ACC>), GRID, BLOCK, 0, stream,  \
                         p, tiles_m, tiles_n);                                                     \
    } else if (p.fmt_a == FP8_E5M2 && p.fmt_b == FP8_E5M2) {                                       \
      hipLaunchKernelGGL((KERNEL<AK, BK, FP8_E5M2, FP8_E5M2, MATH, ACC>), GRID, BLOCK, 0, stream,  \
                         p, tiles_m, tiles_n);                                                     \
    } else {                                                                                       \
      return hipErrorInvalidValue;                                                                 \
    }                                                                                              \
    return hipGetLastError();                                                                      \
  } while (0)

template <bool AK, bool BK, int MATH>
hipError_t launch_pp(const GemmProblem& p, hipStream_t stream) {
  int tiles_m, tiles_n;
  const dim3 grid = tile_grid(p, 256, 256, tiles_m, tiles_n), block(512);
  if (p.accumulate) FP8LIN_FORMAT_DISPATCH(gemm_pp_kernel, grid, block, true);
  FP8LIN_FORMAT_DISPATCH(gemm_pp_kernel, grid, block, false);
}

template <bool AK, bool BK, int MATH>
hipError_t launch_quad(const GemmProblem& p, hipStream_t stream) {
  int tiles_m, tiles_n;
  const dim3 grid = tile_grid(p, 128, 128, tiles_m, tiles_n), block(256);
  if (p.accumulate) FP8LIN_FORMAT_DISPATCH(gemm_quad_kernel, grid, block, true);
  FP8LIN_FORMAT_DISPATCH(gemm_quad_kernel, grid, block, false);
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

// FP8LIN_GEMM_TILE=128 or 256 pins the pipelined kernel's tile (tuning and
// tests); otherwise it is chosen from the shape.
inline int forced_tile() {
  const char* s = std::getenv("FP8LIN_GEMM_TILE");
  if (!s) return 0;
  const int v = std::atoi(s);
  return (v == 128 || v == 256) ? v : 0;
}

// The pipelined kernels need: a contraction that is a whole number of 64-byte
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

// How an output is cut into launches.  The 256x256 tile does twice the MFMA
// work per byte of LDS and global traffic of the 128x128 one, but a launch
// whose tile count is not a multiple of the chip's 256 workgroup slots runs
// its last wave of tiles part-empty.  Candidates: everything in 256x256
// tiles; everything in 128x128 tiles; or a leading block of whole rows
// (split_m) or columns (split_n), a multiple of 256, in 256x256 tiles and the
// rest in 128x128 tiles, as two launches.  The cost is the number of waves of
// tiles, a 128x128 wave counting a third of a 256x256 one (a quarter of the
// work at ~75% of the rate).
struct TilePlan {
  int tile;     // 256 or 128: the tile of the whole output, when not split
  int split_m;  // > 0: rows [0, split_m) in 256x256 tiles, the rest in 128x128
  int split_n;  // > 0: columns [0, split_n) likewise
};

inline double plan_waves(int64_t m, int64_t n, int bm) {
  const int64_t tiles = ((m + bm - 1) / bm) * ((n + bm - 1) / bm);
  const double waves = (double)((tiles + 255) / 256);
  return bm == 256 ? waves : waves / 3.0;
}

// For each whole number w of 256x256 waves below the unsplit count, the head
// is the most whole tile-rows (or tile-columns) that fit in w waves.  Past 64
// waves the last wave's idle slots are under 2% of the work: no split.
inline TilePlan plan_tiles(int m, int n) {
  TilePlan best{256, 0, 0};
  double cost = plan_waves(m, n, 256);
  const double c128 = plan_waves(m, n, 128);
  if (c128 < cost) {
    best = TilePlan{128, 0, 0};
    cost = c128;
  }
  const int64_t tm = (m + 255) / 256, tn = (n + 255) / 256, waves = (tm * tn + 255) / 256;
  if (waves > 64) return best;
  for (int64_t w = 1; w < waves; ++w) {
    const int64_t rows = w * 256 / tn, cols = w * 256 / tm;  // whole tile-rows / -columns
    if (rows >= 1 && rows < tm) {
      const double c = plan_waves(rows * 256, n, 256) + plan_waves(m - rows * 256, n, 128);
      if (c < cost - 1e-9) {
        best = TilePlan{256, (int)(rows * 256), 0};
        cost = c;
      }
    }
    if (cols >= 1 && cols < tn) {
      const double c = plan_waves(m, cols * 256, 256) + plan_waves(m, n - cols * 256, 128);
      if (c < cost - 1e-9) {
        best = TilePlan{256, 0, (int)(cols * 256)};
        cost = c;
      }
    }
  }
  return best;
}

template <bool AK, bool BK, int MATH>
hipError_t launch_math(const GemmProblem& p, hipStream_t stream) {
  if (!pipe_ok<AK, BK>(p))
    return launch_general<AK, BK, MATH == kMathNativeFp8 ? kMathNativeFp8 : kMathExact>(p, stream);
  const int forced = forced_tile();
  const TilePlan plan = forced ? TilePlan{forced, 0, 0} : plan_tiles(p.m, p.n);
  if (plan.split_m > 0 || plan.split_n > 0) {
    // Two launches on the stream, the second on the remaining rows or
    // columns: the same problem with its operand and output pointers moved
    // on (offsets are multiples of 256 elements or rows, so every alignment
    // pipe_ok checked still holds, as does m % 16 and n % 16).
    GemmProblem head = p, rest = p;
    if (plan.split_m > 0) {
      const int64_t s = plan.split_m;
      head.m = plan.split_m;
      rest.m = p.m - plan.split_m;
      rest.a = AK ? p.a + s * p.lda : p.a + s;
      rest.c = p.c + s * p.ldc;
    } else {
      const int64_t s = plan.split_n;
      head.n = plan.split_n;
      rest.n = p.n - plan.split_n;
      rest.b = BK ? p.b + s * p.ldb : p.b + s;
      rest.c = p.c + s;
    }
    if (hipError_t e = launch_pp<AK, BK, MATH>(head, stream)) return e;
    return launch_quad<AK, BK, MATH>(rest, stream);
  }
  if (plan.tile == 256) return launch_pp<AK, BK, MATH>(p, stream);
  return launch_quad<AK, BK, MATH>(p, stream);
}

// Exact products run on the bf16 MFMA when either operand is E5M2 and on the
// fp16 MFMA otherwise: both are exact (every FP8 value is a normal bf16; every
// E4M3 value a normal fp16, every E5M2 value an fp16).  Measured on the
// MI355X: fp16 1-2% ahead for E4M3 x E4M3; with an E5M2 operand the two
// within 0.2-0.7% of each other (bf16 was ~10% ahead while the fp16 path
// widened E5M2 with shifts and masks rather than one byte permutation per two
// codes).  FP8LIN_EXACT_MFMA=f16 or bf16 forces one (tuning and tests).
inline bool exact_on_bf16(const GemmProblem& p) {
  const char* s = std::getenv("FP8LIN_EXACT_MFMA");
  if (s && std::strcmp(s, "bf16") == 0) return true;
  if (s && std::strcmp(s, "f16") == 0) return false;
  return p.fmt_a == FP8_E5M2 || p.fmt_b == FP8_E5M2;
}

template <bool AK, bool BK>
hipError_t launch_layout(const GemmProblem& p, hipStream_t stream) {
  if (p.m <= 0 || p.n <= 0) return hipSuccess;
  if (rows_ok<AK, BK>(p))
    return exact_on_bf16(p) ? launch_rows<kMathExactBf16>(p, stream) : launch_rows<kMathExact>(p, stream);
  if (gemv_ok<AK, BK>(p)) return launch_gemv(p, stream);
  if (p.math == kMathNativeFp8) return launch_math<AK, BK, kMathNativeFp8>(p, stream);
  if (exact_on_bf16(p)) return launch_math<AK, BK, kMathExactBf16>(p, stream);
  return launch_math<AK, BK, kMathExact>(p, stream);
}

#undef FP8LIN_FORMAT_DISPATCH

}  // namespace gemm_detail
}  // namespace fp8lin
