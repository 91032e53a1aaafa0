// The forward product for 1 to 64 rows (a few tokens through a large weight,
// as when a served model decodes a small batch).  The weight streams from HBM
// once; the tiled kernels read it in 64-byte pieces of 16 rows per load and
// reach ~3 TB/s there.  Here the weight's rows arrive through LDS DMA in
// 256-byte runs (each load covers four rows x 256 contiguous bytes), and the
// products run on the exact 16-bit MFMA as in the tiled kernels.
//
// "Training and inference of large language models using 8-bit floating
// point", review page, "Proposed method", bullet 3 (the product of the scaled
// FP8 operands, unscaled after the matmul) and bullet 5 (inference).
//
// One workgroup of eight waves per 32 x CN output columns (CN tiles of 32 rows
// of W) and all M rows (RB blocks of 32).  Stage = 256 contraction bytes: CN
// 32 x 256-byte tiles of W and RB of X (X's rows past M re-read row M - 1 and
// are zeroed in the fragments), SL stages in a ring (2 or 3, chosen by
// launch_rows), SL - 1 in flight.  Wave w multiplies bytes [32w, 32w + 32) of
// every stage (two 32x32x16 MFMAs per row block and column tile) into its own
// partial sums; the eight waves' partial sums meet in LDS and are added in
// wave order, then unscaled once.
//
// Stage order: workgroup b starts at stage 5b mod (K / 256) and wraps.  Where
// W's rows lie a power of two apart (K = 8192), workgroups that walk the
// stages in step read the same offset of many rows at once, which falls into
// few HBM channels (28672 x 8192 weights: 55 us in step, 37 us rotated).  The
// order depends on the shape and the workgroup only: the same bits on every
// call.  Exact arithmetic only: the native FP8 path keeps the tiled kernels,
// whose 64-product groups its error bound assumes.
//
// Part of gemm_pipe.h (included there after the helpers it uses).
#pragma once

namespace fp8lin {
namespace gemm_detail {

constexpr int kRowsMax = 64;                // output rows taken (two blocks of 32)
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

template <int FA, int FB, int MATH, bool ACC, int RB, int SL, int CN>
__global__ __launch_bounds__(kRowsWaves * 64) void gemm_rows_kernel(GemmProblem p) {
  // ring of SL stages: slot s holds W's CN tiles (32 rows each) at
  // s * (CN + RB) * 8 KB and X's RB tiles after them; at the end it holds the
  // eight waves' partial sums, kChunk row blocks (CN * 32 KB each) at a time
  constexpr int kSlot = (CN + RB) * kRowsTile;
  constexpr int kFit = SL * kSlot / (kRowsWaves * 32 * 32 * CN * 4);
  constexpr int kChunk = RB <= kFit ? RB : 1;
  static_assert(kFit >= 1, "partial sums fit the ring");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[SL * kSlot];
  const int lane = (int)threadIdx.x & 63, wave = wave_id();
  const int rl = lane & 31, h = lane >> 5;
  const int n0 = (int)blockIdx.x * 32 * CN;
  const uint32_t ring0 = lds_addr(ring);
  const int nk = p.k / kRowsStage;
  const int rot = (int)((blockIdx.x * 5u) % (uint32_t)max(nk, 1));
  auto issue = [&](int s, int slot) {
    const uint32_t t = ring0 + slot * kSlot;
    const int se = s + rot < nk ? s + rot : s + rot - nk;
#pragma unroll
    for (int cn = 0; cn < CN; ++cn) rows_dma(p.b, p.ldb, n0 + 32 * cn, p.n, se, t + cn * kRowsTile, wave, lane);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) rows_dma(p.a, p.lda, 32 * rb, p.m, se, t + (CN + rb) * kRowsTile, wave, lane);
  };
  // this lane's fragment: logical chunk 2 wave + h of row rl
  const uint32_t frag = rl * kRowsStage + (rows_swz(rl, 2 * wave + h) << 4);

  v16f acc[RB][CN];
  zero_acc(acc);
#pragma unroll
  for (int s = 0; s < SL - 1; ++s)
    if (s < nk) issue(s, s);
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    wait_stages<CN + RB>(min(SL - 2, nk - 1 - kt));
    bare_barrier();
    if (kt + SL - 1 < nk) issue(kt + SL - 1, slot == 0 ? SL - 1 : slot - 1);
    typedef int v4i __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const v4i* lds_v4i;
    const uint32_t t = ring0 + slot * kSlot + opaque(frag);
    v4i w[CN], x[RB];
#pragma unroll
    for (int cn = 0; cn < CN; ++cn) w[cn] = *(lds_v4i)(uintptr_t)(t + cn * kRowsTile);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      x[rb] = *(lds_v4i)(uintptr_t)(t + (CN + rb) * kRowsTile);
      if (32 * rb + rl >= p.m) x[rb] = v4i{0, 0, 0, 0};
    }
    // two 32x32x16 steps over the lane's 16 bytes (8 contraction values each)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if constexpr (MATH == kMathExactBf16) {
        v8bf b[CN];
#pragma unroll
        for (int cn = 0; cn < CN; ++cn) b[cn] = fp8x8_to_bf16<FB>(w[cn][2 * q], w[cn][2 * q + 1]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const v8bf a = fp8x8_to_bf16<FA>(x[rb][2 * q], x[rb][2 * q + 1]);
#pragma unroll
          for (int cn = 0; cn < CN; ++cn)
            acc[rb][cn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[cn], acc[rb][cn], 0, 0, 0);
        }
      } else {
        v8h b[CN];
#pragma unroll
        for (int cn = 0; cn < CN; ++cn) b[cn] = fp8x8_to_f16<FB>(w[cn][2 * q], w[cn][2 * q + 1]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const v8h a = fp8x8_to_f16<FA>(x[rb][2 * q], x[rb][2 * q + 1]);
#pragma unroll
          for (int cn = 0; cn < CN; ++cn)
            acc[rb][cn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[cn], acc[rb][cn], 0, 0, 0);
        }
      }
    }
    slot = slot == SL - 1 ? 0 : slot + 1;
  }

  // every wave's LDS reads are done (their values fed the MFMAs) and no DMA
  // is in flight (the last stage was waited for): the ring takes the partial
  // sums.  32x32 accumulator layout: register r of lane l holds row
  // 8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32.
  const int unscale = -(*p.bias_a + *p.bias_b);
  uint32_t mx = 0;
  float (*part)[kChunk * 32][32 * CN] = reinterpret_cast<float (*)[kChunk * 32][32 * CN]>(ring);
#pragma unroll
  for (int c0 = 0; c0 < RB; c0 += kChunk) {
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < kChunk; ++rb)
#pragma unroll
      for (int cn = 0; cn < CN; ++cn)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          part[wave][32 * rb + 8 * (r >> 2) + 4 * h + (r & 3)][32 * cn + rl] = acc[c0 + rb][cn][r];
    __syncthreads();
#pragma unroll
    for (int o = (int)threadIdx.x; o < kChunk * 32 * 32 * CN; o += kRowsWaves * 64) {
      const int lr = o / (32 * CN), col = o % (32 * CN), row = 32 * c0 + lr;
      float sum = part[0][lr][col];
#pragma unroll
      for (int w2 = 1; w2 < kRowsWaves; ++w2) sum += part[w2][lr][col];
      if (row < p.m && n0 + col < p.n) {
        float* c = p.c + (int64_t)row * p.ldc + n0 + col;
        float v = __builtin_ldexpf(sum, unscale);
        if constexpr (ACC) v = *c + v;
        *c = v;
        mx = max(mx, __float_as_uint(v) & 0x7FFFFFFFu);
      }
    }
  }
  if (p.amax) amax_fold(mx, p.amax);
}

// Whether a product takes this kernel: the forward layout (both operands
// contraction-contiguous), exact arithmetic, 1 to kRowsMax output rows, whole
// 256-byte stages, 16-byte aligned rows, fewer than 2^28 columns.
template <bool AK, bool BK>
bool rows_ok(const GemmProblem& p) {
  if constexpr (!(AK && BK)) {
    return false;
  } else {
    if (p.math == kMathNativeFp8 || p.m < 1 || p.m > kRowsMax || p.n < 1) return false;
    if (p.k % kRowsStage != 0) return false;
    // a dispatch counts its lanes in 32 bits: 512 per 32 columns
    if ((int64_t)((p.n + 31) / 32) * (kRowsWaves * 64) > (int64_t)0xFFFFFFFF) return false;
    auto aligned = [](const void* q, int64_t ld) { return ((uintptr_t)q % 16 == 0) && (ld % 16 == 0); };
    return aligned(p.a, p.lda) && aligned(p.b, p.ldb);
  }
}

template <int MATH, bool ACC, int RB, int SL, int CN = 1>
hipError_t launch_rows_acc(const GemmProblem& p, hipStream_t stream) {
  const dim3 grid((uint32_t)((p.n + 32 * CN - 1) / (32 * CN))), block(kRowsWaves * 64);
#define FP8LIN_ROWS_CASE(FA, FB)                                                                        \
  if (p.fmt_a == FA && p.fmt_b == FB) {                                                                 \
    hipLaunchKernelGGL((gemm_rows_kernel<FA, FB, MATH, ACC, RB, SL, CN>), grid, block, 0, stream, p); \
    return hipGetLastError();                                                                           \
  }
  FP8LIN_ROWS_CASE(FP8_E4M3, FP8_E4M3)
  FP8LIN_ROWS_CASE(FP8_E5M2, FP8_E4M3)
  FP8LIN_ROWS_CASE(FP8_E4M3, FP8_E5M2)
  FP8LIN_ROWS_CASE(FP8_E5M2, FP8_E5M2)
#undef FP8LIN_ROWS_CASE
  return hipErrorInvalidValue;
}

// Up to 32 rows: one row block, three stages (48 KB of LDS, three workgroups
// per CU; four stages, two workgroups per CU, measured 1-3% slower on the 70B
// weights and 10% on 10240 x 8192, whose 320 workgroups leave 64 CUs with two;
// five and six stages slower still).  Two stages (32 KB, five workgroups per
// CU) where a grid of at least 768 workgroups would not fit the CUs at three
// and the rows are few (28672 x 8192 weights at 1, 8, 16 rows: 33.0, 33.6,
// 34.7 against 36.3, 36.0, 36.3 us; 57344 x 8192 at 24 rows 89 against 97;
// from 28 rows mixed: 32768 x 4096 at 32 rows 21.7 against 20.8; with 256 or
// 320 workgroups two stages lose up to 60%).  From 25 rows over 768 or more
// column tiles, two column tiles per workgroup: X's tiles, which every
// workgroup reads, then cost half as much per weight byte (25-32 rows in
// three stages, 72 KB: 28672 x 8192 weights 34.2-34.7 against 36.3-37.0 us,
// 57344 x 8192 91-92 against 98-101).  33 to 64 rows: two row blocks; over
// 768 or more column tiles two column tiles per workgroup in two stages
// (64 KB, two workgroups per CU: 28672 x 8192 at 33 / 64 rows 37.4 / 38.5
// against 44.8 / 48.3 us), else one in three stages (72 KB; two column tiles
// on 256 workgroups or fewer leave CUs idle: 8192 x 28672 at 64 rows 77
// against 49 us; four stages, 96 KB, one workgroup per CU, were slower:
// 28672 x 8192 at 64 rows 58.0 against 47.7 us).
template <int MATH>
hipError_t launch_rows(const GemmProblem& p, hipStream_t stream) {
  const bool wide = p.n >= 768 * 32;
  if (p.m <= 24 && wide)
    return p.accumulate ? launch_rows_acc<MATH, true, 1, 2>(p, stream) : launch_rows_acc<MATH, false, 1, 2>(p, stream);
  if (p.m <= 32) {
    if (wide)
      return p.accumulate ? launch_rows_acc<MATH, true, 1, 3, 2>(p, stream)
                          : launch_rows_acc<MATH, false, 1, 3, 2>(p, stream);
    return p.accumulate ? launch_rows_acc<MATH, true, 1, 3>(p, stream) : launch_rows_acc<MATH, false, 1, 3>(p, stream);
  }
  if (wide)
    return p.accumulate ? launch_rows_acc<MATH, true, 2, 2, 2>(p, stream)
                        : launch_rows_acc<MATH, false, 2, 2, 2>(p, stream);
  return p.accumulate ? launch_rows_acc<MATH, true, 2, 3>(p, stream) : launch_rows_acc<MATH, false, 2, 3>(p, stream);
}

}  // namespace gemm_detail
}  // namespace fp8lin
