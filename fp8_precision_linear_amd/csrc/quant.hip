// Per-tensor amax, compute_bias and scale-then-cast for gfx950.
//
// "Training and inference of large language models using 8-bit floating
// point", review page, "Proposed method", bullets 1-4: a per-tensor maximum
// absolute value, a power-of-two bias from log2(format max / amax) with a
// margin, and a cast of the scaled tensor to E4M3 (weights, activations) or
// E5M2 (gradients); also E3M4, the third format of "Efficient post-training
// quantization with FP8 formats" (summary page), cast only.  Inputs are bf16
// or fp32.  The cast can also fold its own input's amax (for delayed scaling,
// where the bias comes from the previous step's amax).
//
// All three are HBM-streaming kernels: 16-byte loads and stores per lane,
// grid-stride loops, several loads in flight per lane.  amax reduces on the
// integer magnitude bits (for non-negative IEEE values integer order is value
// order, with NaN above inf), so the result is exact and independent of the
// reduction order: wave shuffle, then LDS across the block's waves, then one
// atomicMax per block.
#include <cstdlib>
#include <cstring>

#include <type_traits>

#include "internal.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Launch shapes and cache hints measured on MI355X over 128 MiB and 448 MiB
// bf16 tensors, both cold (after a cache flush) and right after amax:
//  * amax peaks with one 256-lane block per CU and 8 loads in flight per lane
//    (more blocks add contention on the single atomicMax target);
//  * the cast peaks with one 16-element unit per lane per iteration over a
//    grid of up to 32768 blocks (every lane's two loads in flight at once):
//    6.2 TB/s cold and 6.6 TB/s warm on 128 MiB, 6.4 / 6.8 TB/s on 448 MiB,
//    against 4.7-5.4 cold with four units per lane over 4096 blocks;
//  * amax and cast read with non-temporal loads, which do not allocate in the
//    Infinity Cache: when the cache holds dirty lines (as after a GEMM has
//    written its fp32 output) ordinary loads pay for writing them back (amax
//    2.4 against 5.5 TB/s on 128 MiB), and in the full inference step this
//    choice gives the shortest amax + bias + cast of all the combinations
//    measured; the FP8 codes are stored ordinarily (faster than streaming
//    stores in every case measured).
//  FP8LIN_AMAX_HINT / FP8LIN_CAST_HINT = cached | nt override the load hint
//  (tuning).
constexpr int kAmaxUnroll = 8;
constexpr int kAmaxMaxBlocks = 256;
constexpr int kCastUnitsPerLane = 1;  // launch shape: units per lane
constexpr int kCastMaxBlocks = 32768;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte accesses, non-temporal (NT: streaming, every byte touched once) or
// ordinary (cached).
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *p;
  }
}

template <bool NT>
__device__ __forceinline__ void store16(uint4 v, uint4* p) {
  if constexpr (NT) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  } else {
    *p = v;
  }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Block-wide max of v, folded into *out with one atomic per block.
__device__ __forceinline__ void block_max_to(uint32_t v, uint32_t* out) {
  __shared__ uint32_t part[kWaves];
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = part[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = max(m, part[w]);
    atomicMax(out, m);
  }
}

__global__ void amax_clear_kernel(uint32_t* out) { *out = 0u; }

// bf16: each 16-byte vector holds 8 values; the running max is kept as two
// packed 16-bit magnitudes (sign bits masked off).
__device__ __forceinline__ u16x2 bf16_mag2(uint32_t w) {
  uint32_t m = w & 0x7FFF7FFFu;
  return *reinterpret_cast<u16x2*>(&m);
}

__device__ __forceinline__ u16x2 vmax_bf16(u16x2 acc, uint4 v) {
  acc = __builtin_elementwise_max(acc, bf16_mag2(v.x));
  acc = __builtin_elementwise_max(acc, bf16_mag2(v.y));
  acc = __builtin_elementwise_max(acc, bf16_mag2(v.z));
  acc = __builtin_elementwise_max(acc, bf16_mag2(v.w));
  return acc;
}

// The lane's largest bf16 magnitude over the tensor's 8-element vectors that
// block blk of nblk covers (grid-stride), plus block 0's share of the tail.
template <bool NT>
__device__ __forceinline__ uint32_t amax_bf16_body(const uint4* __restrict__ x, int64_t nvec,
                                                   const uint16_t* __restrict__ tail, int ntail,
                                                   int64_t blk, int64_t nblk) {
  u16x2 acc = {0, 0};
  const int64_t stride = nblk * kThreads;
  int64_t i = blk * kThreads + threadIdx.x;
  for (; i + (kAmaxUnroll - 1) * stride < nvec; i += kAmaxUnroll * stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) v[u] = load16<NT>(&x[i + u * stride]);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) acc = vmax_bf16(acc, v[u]);
  }
  for (; i < nvec; i += stride) acc = vmax_bf16(acc, load16<NT>(&x[i]));
  uint32_t m = max((uint32_t)acc.x, (uint32_t)acc.y);
  if (blk == 0 && (int)threadIdx.x < ntail) m = max(m, (uint32_t)(tail[threadIdx.x] & 0x7FFFu));
  return m << 16;  // bf16 magnitude widened to fp32 bits
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void amax_bf16_kernel(const uint4* __restrict__ x,
                                                             int64_t nvec,
                                                             const uint16_t* __restrict__ tail,
                                                             int ntail, uint32_t* out) {
  block_max_to(amax_bf16_body<NT>(x, nvec, tail, ntail, blockIdx.x, gridDim.x), out);
}

__device__ __forceinline__ uint32_t vmax_f32(uint32_t acc, uint4 v) {
  acc = max(acc, max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu));
  acc = max(acc, max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
  return acc;
}

template <bool NT>
__device__ __forceinline__ uint32_t amax_f32_body(const uint4* __restrict__ x, int64_t nvec,
                                                  const uint32_t* __restrict__ tail, int ntail,
                                                  int64_t blk, int64_t nblk) {
  uint32_t m = 0;
  const int64_t stride = nblk * kThreads;
  int64_t i = blk * kThreads + threadIdx.x;
  for (; i + (kAmaxUnroll - 1) * stride < nvec; i += kAmaxUnroll * stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) v[u] = load16<NT>(&x[i + u * stride]);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = vmax_f32(m, v[u]);
  }
  for (; i < nvec; i += stride) m = vmax_f32(m, load16<NT>(&x[i]));
  if (blk == 0 && (int)threadIdx.x < ntail) m = max(m, tail[threadIdx.x] & 0x7FFFFFFFu);
  return m;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void amax_f32_kernel(const uint4* __restrict__ x,
                                                            int64_t nvec,
                                                            const uint32_t* __restrict__ tail,
                                                            int ntail, uint32_t* out) {
  block_max_to(amax_f32_body<NT>(x, nvec, tail, ntail, blockIdx.x, gridDim.x), out);
}

// ---------------------------------------------------------------- bias
// floor(log2(fmt_max / A)) - margin with fmt_max = t * 2^emax, t = 1.75 for
// E4M3 (448) and E5M2 (57344), 1.875 for E3M4 (30).  Writing A = (1 + f) * 2^e
// with f in [0, 1): fmt_max / A = t / (1 + f) * 2^(emax - e) and t / (1 + f)
// lies in (t / 2, t], so its floor(log2) is 0 when 1 + f <= t (fraction field
// <= 0x600000, resp. 0x700000) and -1 otherwise.
__device__ __forceinline__ int32_t bias_from_amax_bits(uint32_t a, int fmt, int32_t margin) {
  if (a == 0u || a >= 0x7F800000u) return 0;  // zero, inf, NaN (or a negative input)
  int e;
  uint32_t frac;
  if ((a >> 23) == 0u) {  // subnormal: normalise on the leading one
    const int p = 31 - __clz(a);
    e = p - 149;
    frac = (a << (23 - p)) & 0x7FFFFFu;
  } else {
    e = (int)(a >> 23) - 127;
    frac = a & 0x7FFFFFu;
  }
  const int emax = fmt == FP8_E4M3 ? 8 : (fmt == FP8_E5M2 ? 15 : 4);
  const uint32_t tfrac = fmt == FP8_E3M4 ? 0x700000u : 0x600000u;
  return emax - e - (frac > tfrac ? 1 : 0) - margin;
}

__global__ void bias_kernel(const uint32_t* __restrict__ amax, int fmt, int32_t margin,
                            int32_t* __restrict__ bias) {
  *bias = bias_from_amax_bits(*amax, fmt, margin);
}

// Delayed scaling of an empty tensor: the bias from the previous amax, then
// the amax of nothing (0).
__global__ void delayed_empty_kernel(uint32_t* amax, int fmt, int32_t margin, int32_t* bias) {
  *bias = bias_from_amax_bits(*amax, fmt, margin);
  *amax = 0u;
}

// Where a cast takes its bias from: the int32 at `bias`, or -- the whole
// quantisation in one call -- the amax word the amax kernel just wrote, turned
// into the bias in every block exactly as bias_kernel does; lane 0 of block 0
// then also stores it at `bias_out` for the products that follow.
struct BiasArg {
  const int32_t* bias;    // used when amax is null
  const uint32_t* amax;   // non-null: the bias is derived from *amax and margin
  int32_t* bias_out;      // with amax: receives the derived bias
  int32_t margin;
};

template <int FMT>
__device__ __forceinline__ int32_t load_bias(const BiasArg& a) {
  return a.amax ? bias_from_amax_bits(*a.amax, FMT, a.margin) : *a.bias;
}

template <int FMT>
__device__ __forceinline__ void store_derived_bias(const BiasArg& a, int64_t blk) {
  if (a.amax && blk == 0 && threadIdx.x == 0) *a.bias_out = load_bias<FMT>(a);
}

// ---------------------------------------------------------------- cast
// x * 2^b is formed exactly with ldexp: fp32 denormals are kept (the kernels
// run with denormal mode "preserve"), results at or above 2^-126 are exact,
// smaller ones cast to a signed zero in both formats anyway, and results past
// the fp32 range become inf, which saturates like any value above fmt_max.
// The magnitude bits a of the scaled value are then rounded to the format:
//   normal range    round-to-nearest-even on the dropped fraction bits, the
//                   exponent re-biased by one constant (a carry moves into the
//                   next binade on its own);
//   subnormal range adding 2^(23 + emin - mbits) -- the power of two whose
//                   fp32 ulp is the format's smallest subnormal -- lets the
//                   fp32 adder round to that quantum; the integer difference
//                   of the bit patterns is the code;
// then saturation at the largest finite code and NaN -> 0x7F, sign copied.
template <int FMT>
__device__ __forceinline__ uint32_t fp8_code(uint32_t xbits, int32_t b) {
  const uint32_t vb = __float_as_uint(__builtin_ldexpf(__uint_as_float(xbits), b));
  const uint32_t a = vb & 0x7FFFFFFFu;
  uint32_t code;
  if constexpr (FMT == FP8_E4M3) {
    // normal: code = (fp32 exponent - 120) * 8 + top 3 fraction bits, rounded
    const uint32_t nrm = (a + (0x7FFFFu - 0x3C000000u) + ((a >> 20) & 1u)) >> 20;
    // subnormal (|v| < 2^-6): the ulp of 2^14 in fp32 is 2^-9
    const uint32_t sub = __float_as_uint(__uint_as_float(a) + 16384.0f) - 0x46800000u;
    code = a < 0x3C800000u ? sub : nrm;
    code = min(code, 0x7Eu);
  } else if constexpr (FMT == FP8_E5M2) {
    // normal: code = (fp32 exponent - 112) * 4 + top 2 fraction bits, rounded
    const uint32_t nrm = (a + (0xFFFFFu - 0x38000000u) + ((a >> 21) & 1u)) >> 21;
    // subnormal (|v| < 2^-14): the ulp of 2^7 in fp32 is 2^-16
    const uint32_t sub = __float_as_uint(__uint_as_float(a) + 128.0f) - 0x43000000u;
    code = a < 0x38800000u ? sub : nrm;
    code = min(code, 0x7Bu);
  } else {
    static_assert(FMT == FP8_E3M4, "unknown format");
    // normal: code = (fp32 exponent - 124) * 16 + top 4 fraction bits, rounded
    const uint32_t nrm = (a + (0x3FFFFu - 0x3E000000u) + ((a >> 19) & 1u)) >> 19;
    // subnormal (|v| < 2^-2): the ulp of 2^17 in fp32 is 2^-6
    const uint32_t sub = __float_as_uint(__uint_as_float(a) + 131072.0f) - 0x48000000u;
    code = a < 0x3E800000u ? sub : nrm;
    code = min(code, 0x7Eu);  // 30; the code above it is NaN
  }
  code = a > 0x7F800000u ? 0x7Fu : code;
  return code | ((vb >> 24) & 0x80u);
}

template <int FMT>
__device__ __forceinline__ uint32_t pack4_bf16(uint32_t w0, uint32_t w1, int32_t b) {
  const uint32_t c0 = fp8_code<FMT>(w0 << 16, b);
  const uint32_t c1 = fp8_code<FMT>(w0 & 0xFFFF0000u, b);
  const uint32_t c2 = fp8_code<FMT>(w1 << 16, b);
  const uint32_t c3 = fp8_code<FMT>(w1 & 0xFFFF0000u, b);
  return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

template <int FMT>
__device__ __forceinline__ uint32_t pack4_f32(uint4 v, int32_t b) {
  return fp8_code<FMT>(v.x, b) | (fp8_code<FMT>(v.y, b) << 8) | (fp8_code<FMT>(v.z, b) << 16) |
         (fp8_code<FMT>(v.w, b) << 24);
}

// ---------------------------------------------------------------- cast, hardware conversion
// gfx950's v_cvt_scalef32_pk_{fp8,bf8}_bf16 converts two bf16 values x to the
// FP8 codes of x / scale with round-to-nearest-even.  Measured against the
// rounding defined above on every bf16 pattern and every scale 2^k,
// k = -126..127: bit-identical for every finite input whose scaled value does
// not exceed the format's largest finite value; beyond it the instruction
// returns NaN / inf codes instead of saturating, and its NaN and inf codes
// differ from the ones defined here.  So, with scale = 2^-b (a normal float
// for b in [-127, 126]):
//  * finite inputs are first clamped in magnitude to fmt_max * 2^-b (a packed
//    16-bit integer min on the magnitude bits: for non-negative IEEE values
//    integer order is value order), which turns overflow into exactly the
//    saturation the rounding above performs (every value at or beyond
//    fmt_max rounds to the largest finite code);
//  * a unit holding any inf or NaN is redone with fp8_code.
// E3M4 has no such conversion and always takes fp8_code.
constexpr int kHwBiasMin = -127, kHwBiasMax = 126;
template <int FMT>
constexpr bool kHwConvert = FMT == FP8_E4M3 || FMT == FP8_E5M2;

typedef short hw_v2s __attribute__((ext_vector_type(2)));
typedef __bf16 hw_v2bf __attribute__((ext_vector_type(2)));

// bf16 magnitude bits of min(fmt_max * 2^-b, largest finite bf16), twice.
// fmt_max = 1.75 * 2^emax has bf16 fraction bits 0x60.
template <int FMT>
__device__ __forceinline__ uint32_t hw_bound2(int32_t b) {
  static_assert(kHwConvert<FMT>, "no hardware conversion for this format");
  const int efield = (FMT == FP8_E4M3 ? 8 : 15) + 127 - b;
  const uint32_t m = efield >= 255 ? 0x7F7Fu : (((uint32_t)efield << 7) | 0x60u);
  return m | (m << 16);
}

// Four bf16 values (two dwords) -> four codes.  mx accumulates the largest
// magnitude seen (per 16-bit half) for the non-finite check.
template <int FMT>
__device__ __forceinline__ uint32_t pack4_bf16_hw(uint32_t w0, uint32_t w1, uint32_t bound2,
                                                  float scale, u16x2& mx) {
  const u16x2 m0 = bf16_mag2(w0), m1 = bf16_mag2(w1), bd = *reinterpret_cast<u16x2*>(&bound2);
  mx = __builtin_elementwise_max(mx, __builtin_elementwise_max(m0, m1));
  const u16x2 c0 = __builtin_elementwise_min(m0, bd), c1 = __builtin_elementwise_min(m1, bd);
  const uint32_t x0 = (w0 & 0x80008000u) | __builtin_bit_cast(uint32_t, c0);
  const uint32_t x1 = (w1 & 0x80008000u) | __builtin_bit_cast(uint32_t, c1);
  hw_v2s r = {0, 0};
  if constexpr (FMT == FP8_E4M3) {
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(hw_v2bf, x0), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(hw_v2bf, x1), scale, true);
  } else {
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(hw_v2bf, x0), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(hw_v2bf, x1), scale, true);
  }
  return __builtin_bit_cast(uint32_t, r);
}

// One unit (16 bf16 values in lo, hi) with the hardware conversion, or with
// fp8_code if it holds an inf or NaN.
template <int FMT>
__device__ __forceinline__ uint4 cast_unit_hw(uint4 lo, uint4 hi, int32_t b, uint32_t bound2,
                                              float scale) {
  u16x2 mx = {0, 0};
  uint4 o;
  o.x = pack4_bf16_hw<FMT>(lo.x, lo.y, bound2, scale, mx);
  o.y = pack4_bf16_hw<FMT>(lo.z, lo.w, bound2, scale, mx);
  o.z = pack4_bf16_hw<FMT>(hi.x, hi.y, bound2, scale, mx);
  o.w = pack4_bf16_hw<FMT>(hi.z, hi.w, bound2, scale, mx);
  if (max(mx.x, mx.y) >= 0x7F80u) {  // inf or NaN present
    o.x = pack4_bf16<FMT>(lo.x, lo.y, b);
    o.y = pack4_bf16<FMT>(lo.z, lo.w, b);
    o.z = pack4_bf16<FMT>(hi.x, hi.y, b);
    o.w = pack4_bf16<FMT>(hi.z, hi.w, b);
  }
  return o;
}

// fp32 magnitude bits of min(fmt_max * 2^-b, largest finite fp32); fmt_max =
// 1.75 * 2^emax has fp32 fraction bits 0x600000.
template <int FMT>
__device__ __forceinline__ uint32_t hw_bound_f32(int32_t b) {
  static_assert(kHwConvert<FMT>, "no hardware conversion for this format");
  const int efield = (FMT == FP8_E4M3 ? 8 : 15) + 127 - b;
  return efield >= 255 ? 0x7F7FFFFFu : (((uint32_t)efield << 23) | 0x600000u);
}

// Four fp32 values -> four codes with v_cvt_scalef32_pk_{fp8,bf8}_f32, the
// magnitudes clamped to fmt_max * 2^-b first (as for bf16 inputs); mx keeps
// the largest magnitude seen, for the non-finite check.
template <int FMT>
__device__ __forceinline__ uint32_t pack4_f32_hw(uint4 v, uint32_t bound, float scale, uint32_t& mx) {
  const uint32_t m0 = v.x & 0x7FFFFFFFu, m1 = v.y & 0x7FFFFFFFu;
  const uint32_t m2 = v.z & 0x7FFFFFFFu, m3 = v.w & 0x7FFFFFFFu;
  mx = max(mx, max(max(m0, m1), max(m2, m3)));
  const float c0 = __uint_as_float((v.x & 0x80000000u) | min(m0, bound));
  const float c1 = __uint_as_float((v.y & 0x80000000u) | min(m1, bound));
  const float c2 = __uint_as_float((v.z & 0x80000000u) | min(m2, bound));
  const float c3 = __uint_as_float((v.w & 0x80000000u) | min(m3, bound));
  hw_v2s r = {0, 0};
  if constexpr (FMT == FP8_E4M3) {
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c0, c1, scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c2, c3, scale, true);
  } else {
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, c0, c1, scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, c2, c3, scale, true);
  }
  return __builtin_bit_cast(uint32_t, r);
}

template <int FMT>
__device__ __forceinline__ uint4 cast_unit_sw(uint4 lo, uint4 hi, int32_t b) {
  uint4 o;
  o.x = pack4_bf16<FMT>(lo.x, lo.y, b);
  o.y = pack4_bf16<FMT>(lo.z, lo.w, b);
  o.z = pack4_bf16<FMT>(hi.x, hi.y, b);
  o.w = pack4_bf16<FMT>(hi.z, hi.w, b);
  return o;
}

// One unit = 16 elements -> one 16-byte store.  The data loads do not depend
// on the bias, so they are issued before the bias load has returned; the
// choice between the hardware conversion (bias in [kHwBiasMin, kHwBiasMax],
// E4M3 and E5M2) and fp8_code is a wave-uniform branch per unit after them.
// With AMAX the lane's largest input magnitude (bf16 bits) is returned too.
template <int FMT, bool NT, bool AMAX, int TPB = kThreads>
__device__ __forceinline__ uint32_t cast_bf16_body(const uint4* __restrict__ x, int64_t nunit,
                                                   const BiasArg& bias, uint4* __restrict__ y,
                                                   int64_t blk, int64_t nblk) {
  const int64_t stride = nblk * TPB;
  int64_t i = blk * TPB + threadIdx.x;
  if (i >= nunit) return 0u;
  u16x2 acc = {0, 0};
  uint4 lo = load16<NT>(&x[2 * i]), hi = load16<NT>(&x[2 * i + 1]);
  const int32_t b = load_bias<FMT>(bias);
  const bool hw = kHwConvert<FMT> && b >= kHwBiasMin && b <= kHwBiasMax;
  uint32_t bound2 = 0;
  if constexpr (kHwConvert<FMT>) bound2 = hw_bound2<FMT>(b);
  const float scale = __builtin_ldexpf(1.0f, hw ? -b : 0);
  for (;;) {
    const int64_t next = i + stride;
    uint4 nlo = lo, nhi = hi;
    if (next < nunit) {  // the next unit's loads in flight during this one's conversion
      nlo = load16<NT>(&x[2 * next]);
      nhi = load16<NT>(&x[2 * next + 1]);
    }
    uint4 o;
    if constexpr (kHwConvert<FMT>)
      o = hw ? cast_unit_hw<FMT>(lo, hi, b, bound2, scale) : cast_unit_sw<FMT>(lo, hi, b);
    else
      o = cast_unit_sw<FMT>(lo, hi, b);
    store16<false>(o, &y[i]);
    if constexpr (AMAX) acc = vmax_bf16(vmax_bf16(acc, lo), hi);
    if (next >= nunit) break;
    i = next;
    lo = nlo;
    hi = nhi;
  }
  return max((uint32_t)acc.x, (uint32_t)acc.y);
}

// Block blk of nblk casting a bf16 tensor: its units, the derived bias (block
// 0), block 0's share of the tail; returns the lane's largest input magnitude
// (fp32 bits) when AMAX.
template <int FMT, bool NT, bool AMAX, int TPB = kThreads>
__device__ __forceinline__ uint32_t cast_bf16_whole(const uint4* __restrict__ x, int64_t nunit,
                                                    const BiasArg& bias, uint4* __restrict__ y,
                                                    const uint16_t* __restrict__ tail_x,
                                                    uint8_t* __restrict__ tail_y, int ntail,
                                                    int64_t blk, int64_t nblk) {
  uint32_t m = cast_bf16_body<FMT, NT, AMAX, TPB>(x, nunit, bias, y, blk, nblk);
  store_derived_bias<FMT>(bias, blk);
  if (blk == 0 && (int)threadIdx.x < ntail) {
    const uint32_t w = tail_x[threadIdx.x];
    tail_y[threadIdx.x] = (uint8_t)fp8_code<FMT>(w << 16, load_bias<FMT>(bias));
    m = max(m, w & 0x7FFFu);
  }
  return m << 16;
}

template <int FMT, bool NT>
__global__ __launch_bounds__(kThreads) void cast_bf16_kernel(const uint4* __restrict__ x,
                                                             int64_t nunit, BiasArg bias,
                                                             uint4* __restrict__ y,
                                                             const uint16_t* __restrict__ tail_x,
                                                             uint8_t* __restrict__ tail_y,
                                                             int ntail) {
  cast_bf16_whole<FMT, NT, false>(x, nunit, bias, y, tail_x, tail_y, ntail, blockIdx.x, gridDim.x);
}

// fp32 input: a wave takes chunks of kF32Chunk consecutive elements; load k
// of lane l reads elements [256k + 4l, +4) of the chunk, so every load
// instruction covers 1 KiB of consecutive bytes (16 bytes per lane, lane-
// contiguous 64-byte runs left each instruction striding and measured 4.2 TB/s
// on MI355X over 90M elements, against 6.4 TB/s this way), and the four codes
// go out as one dword at the same position of the output.  Groups of four
// holding an inf or NaN take fp8_code.  Elements past the last whole chunk
// (fewer than kF32Chunk) are cast one per lane by block 0.
constexpr int kF32Loads = 4;
constexpr int64_t kF32Chunk = 256 * kF32Loads;

template <int FMT>
__device__ __forceinline__ uint32_t cast4_f32(uint4 v, bool hw, int32_t b, uint32_t bound, float scale) {
  if constexpr (kHwConvert<FMT>) {
    if (hw) {
      uint32_t mx = 0;
      const uint32_t o = pack4_f32_hw<FMT>(v, bound, scale, mx);
      if (mx < 0x7F800000u) return o;
    }
  }
  return pack4_f32<FMT>(v, b);
}

template <int FMT, bool NT, bool AMAX, int TPB = kThreads>
__device__ __forceinline__ uint32_t cast_f32_whole(const uint4* __restrict__ x, int64_t nchunk,
                                                   const BiasArg& bias, uint32_t* __restrict__ y,
                                                   const uint32_t* __restrict__ tail_x,
                                                   uint8_t* __restrict__ tail_y, int ntail,
                                                   int64_t blk, int64_t nblk) {
  store_derived_bias<FMT>(bias, blk);
  const int32_t b = load_bias<FMT>(bias);
  const bool hw = kHwConvert<FMT> && b >= kHwBiasMin && b <= kHwBiasMax;
  uint32_t bound = 0;
  if constexpr (kHwConvert<FMT>) bound = hw_bound_f32<FMT>(b);
  const float scale = __builtin_ldexpf(1.0f, hw ? -b : 0);
  const int lane = threadIdx.x & 63;
  const int64_t wstride = nblk * (TPB / 64);
  uint32_t m = 0;
  for (int64_t w = blk * (TPB / 64) + (threadIdx.x >> 6); w < nchunk; w += wstride) {
    const int64_t q = w * (kF32Chunk / 4);  // the chunk's first 16-byte group
    uint4 v[kF32Loads];
#pragma unroll
    for (int k = 0; k < kF32Loads; ++k) v[k] = load16<NT>(&x[q + 64 * k + lane]);
#pragma unroll
    for (int k = 0; k < kF32Loads; ++k) {
      y[q + 64 * k + lane] = cast4_f32<FMT>(v[k], hw, b, bound, scale);
      if constexpr (AMAX) m = vmax_f32(m, v[k]);
    }
  }
  if (blk == 0)
    for (int i = threadIdx.x; i < ntail; i += TPB) {
      tail_y[i] = (uint8_t)fp8_code<FMT>(tail_x[i], b);
      m = max(m, tail_x[i] & 0x7FFFFFFFu);
    }
  return m;
}

template <int FMT, bool NT>
__global__ __launch_bounds__(kThreads) void cast_f32_kernel(const uint4* __restrict__ x,
                                                            int64_t nchunk, BiasArg bias,
                                                            uint32_t* __restrict__ y,
                                                            const uint32_t* __restrict__ tail_x,
                                                            uint8_t* __restrict__ tail_y,
                                                            int ntail) {
  cast_f32_whole<FMT, NT, false>(x, nchunk, bias, y, tail_x, tail_y, ntail, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------- cast + amax
// The cast that also returns max |x| takes two launches and no atomics:
//  * the main cast covers all of the input but a last stretch; each of its
//    blocks stores its largest input magnitude as one word in the bytes of y
//    that the stretch's codes will occupy -- bf16: the plain cast's launch
//    shape (256-lane blocks, one 16-element unit per lane) and 16-bit words
//    (a bf16 magnitude); fp32: 1024-lane blocks, one 1024-element chunk per
//    wave, 32-bit words.  The stretch is the fewest whole units / chunks
//    whose codes hold every word;
//  * one 1024-lane block then loads the words and, only once every lane holds
//    its share of them, casts the stretch and the tail over them and stores
//    the maximum at *amax.
// No block waits at its end for an atomic on one shared word (atomics per
// block measured 40 us against the plain cast's 31.5 on 128 MiB), and the
// result is max |x| over every element, the same integer maximum as
// fp8_amax's.  With delayed scaling in one call the bias comes from the amax
// word itself (the previous step's): every block of both launches derives it
// from that word, and only the last block overwrites the word, at its very
// end, after a barrier that every lane reaches with the bias derived.
constexpr int kLastThreads = 1024;
constexpr int kPartMaxBlocksBf16 = 32768;  // 64 KiB of 16-bit words at most
constexpr int kPartThreadsF32 = 1024;
constexpr int kPartMaxBlocksF32 = 8192;    // 32 KiB of 32-bit words at most
constexpr int64_t kPartSmallUnits = 8192;  // bf16: up to 131072 elements in the last block alone
constexpr int64_t kPartSmallChunks = 64;   // fp32: up to 65536 (+ 1023) elements likewise

// Block-wide max of v (TPB lanes); lane 0 passes it to store(m).
template <int TPB, typename Store>
__device__ __forceinline__ void block_max_then(uint32_t v, Store&& store) {
  __shared__ uint32_t part[TPB / 64];
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = part[0];
#pragma unroll
    for (int w = 1; w < TPB / 64; ++w) m = max(m, part[w]);
    store(m);
  }
}

// The largest of the nwords words (W bits each, W = 16 or 32) the main cast
// left at `words`, read as 32-bit loads, all in flight at once (at most
// kMax words).  Every load is complete -- its value reduced into the lane's
// register -- before the block's barrier, so that no store after it can
// overtake a load of the same address.
template <int W, int kMax>
__device__ __forceinline__ uint32_t words_max(const uint32_t* words, int nwords) {
  constexpr int kPerWord = 32 / W;
  constexpr int kPerLane = kMax / kPerWord / kLastThreads;
  const int nloads = (nwords + kPerWord - 1) / kPerWord;
  uint32_t m = 0;
  {
    uint32_t v[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      v[k] = 0u;
      if (k * kLastThreads < nloads)  // (uniform) lanes past the last load re-read it, count 0
        v[k] = words[min((int)threadIdx.x + k * kLastThreads, nloads - 1)];
    }
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
      const int i = (int)threadIdx.x + k * kLastThreads;
      if constexpr (W == 16) {  // the high half of the last load may lie past the last word
        const uint32_t lo = i < nloads ? (v[k] & 0xFFFFu) : 0u;
        const uint32_t hi = 2 * i + 1 < nwords ? (v[k] >> 16) : 0u;
        m = max(m, max(lo, hi) << 16);  // bf16 magnitude widened to fp32 bits
      } else {
        m = max(m, i < nloads ? v[k] : 0u);
      }
    }
  }
  asm volatile("" : "+v"(m));  // m (hence every load) complete before the barrier
  __syncthreads();
  return m;
}

template <int FMT, bool NT>
__global__ __launch_bounds__(kThreads) void cast_part_bf16_kernel(const uint4* __restrict__ x,
                                                                  int64_t nunit, BiasArg bias,
                                                                  uint4* __restrict__ y,
                                                                  uint16_t* words) {
  const uint32_t m = cast_bf16_body<FMT, NT, true>(x, nunit, bias, y, blockIdx.x, gridDim.x);
  store_derived_bias<FMT>(bias, blockIdx.x);
  block_max_then<kThreads>(m, [&](uint32_t b) { words[blockIdx.x] = (uint16_t)b; });
}

// x, y: the stretch's first unit; nunit (<= kPartSmallUnits): its units.
// The stretch's input is loaded first, all of it at once (at most
// kLastUnits units per lane), so that its latency overlaps the words'.
constexpr int kLastUnits = (int)(kPartSmallUnits / kLastThreads);
static_assert(kPartMaxBlocksBf16 / 8 <= kPartSmallUnits, "the stretch fits the last block");

template <int FMT, bool NT>
__global__ __launch_bounds__(kLastThreads) void cast_last_bf16_kernel(
    const uint4* __restrict__ x, int nunit, BiasArg bias, uint4* __restrict__ y,
    const uint32_t* words, int nwords, const uint16_t* __restrict__ tail_x,
    uint8_t* __restrict__ tail_y, int ntail, uint32_t* amax) {
  const int t = (int)threadIdx.x;
  uint4 lo[kLastUnits], hi[kLastUnits];
#pragma unroll
  for (int u = 0; u < kLastUnits; ++u) {
    if (u * kLastThreads < nunit) {  // (uniform) lanes past the last unit re-read it, unused
      const int i = min(t + u * kLastThreads, nunit - 1);
      lo[u] = load16<NT>(&x[2 * i]);
      hi[u] = load16<NT>(&x[2 * i + 1]);
    }
  }
  const uint32_t tw = t < ntail ? tail_x[t] : 0u;
  uint32_t m = words_max<16, kPartMaxBlocksBf16>(words, nwords);  // then the barrier
  const int32_t b = load_bias<FMT>(bias);
  store_derived_bias<FMT>(bias, 0);
  const bool hw = kHwConvert<FMT> && b >= kHwBiasMin && b <= kHwBiasMax;
  uint32_t bound2 = 0;
  if constexpr (kHwConvert<FMT>) bound2 = hw_bound2<FMT>(b);
  const float scale = __builtin_ldexpf(1.0f, hw ? -b : 0);
  u16x2 acc = {0, 0};
#pragma unroll
  for (int u = 0; u < kLastUnits; ++u) {
    const int i = t + u * kLastThreads;
    if (i < nunit) {
      uint4 o;
      if constexpr (kHwConvert<FMT>)
        o = hw ? cast_unit_hw<FMT>(lo[u], hi[u], b, bound2, scale) : cast_unit_sw<FMT>(lo[u], hi[u], b);
      else
        o = cast_unit_sw<FMT>(lo[u], hi[u], b);
      y[i] = o;
      acc = vmax_bf16(vmax_bf16(acc, lo[u]), hi[u]);
    }
  }
  if (t < ntail) {
    tail_y[t] = (uint8_t)fp8_code<FMT>(tw << 16, b);
    acc.x = max(acc.x, (unsigned short)(tw & 0x7FFFu));
  }
  m = max(m, (uint32_t)max(acc.x, acc.y) << 16);
  __builtin_amdgcn_s_waitcnt(0);  // every load of this wave (the amax word's too) has returned
  block_max_then<kLastThreads>(m, [&](uint32_t v) { *amax = v; });
}

template <int FMT, bool NT>
__global__ __launch_bounds__(kPartThreadsF32) void cast_part_f32_kernel(const uint4* __restrict__ x,
                                                                        int64_t nchunk, BiasArg bias,
                                                                        uint32_t* __restrict__ y,
                                                                        uint32_t* words) {
  const uint32_t m = cast_f32_whole<FMT, NT, true, kPartThreadsF32>(x, nchunk, bias, y, nullptr,
                                                                     nullptr, 0, blockIdx.x, gridDim.x);
  block_max_then<kPartThreadsF32>(m, [&](uint32_t b) { words[blockIdx.x] = b; });
}

template <int FMT, bool NT>
__global__ __launch_bounds__(kLastThreads) void cast_last_f32_kernel(
    const uint4* __restrict__ x, int64_t nchunk, BiasArg bias, uint32_t* __restrict__ y,
    const uint32_t* words, int nwords, const uint32_t* __restrict__ rest_x,
    uint8_t* __restrict__ rest_y, int nrest, uint32_t* amax) {
  uint32_t m = words_max<32, kPartMaxBlocksF32>(words, nwords);
  m = max(m, cast_f32_whole<FMT, NT, true, kLastThreads>(x, nchunk, bias, y, rest_x, rest_y, nrest, 0, 1));
  __builtin_amdgcn_s_waitcnt(0);  // every load of this wave (the amax word's too) has returned
  block_max_then<kLastThreads>(m, [&](uint32_t b) { *amax = b; });
}

// Grid size: `per_lane` units of work per lane of `lanes`-unit blocks, between
// 1 and `cap` blocks.
int stream_blocks_of(int64_t units, int64_t per_lane, int64_t cap, int64_t lanes) {
  const int64_t want = (units + per_lane * lanes - 1) / (per_lane * lanes);
  return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

int stream_blocks(int64_t units, int64_t per_lane, int64_t cap) {
  return stream_blocks_of(units, per_lane, cap, kThreads);
}

// ---------------------------------------------------------------- quantisation in one workgroup
// A small tensor's whole quantisation -- amax, bias, cast -- in one launch of
// one 1024-lane workgroup: the amax is reduced over the workgroup (wave
// shuffles, then LDS), lane 0 stores it and the bias derived from it, and the
// cast re-reads the input (from L2: the tensor was just read).  The results
// are those of the separate amax, bias and cast kernels, bit for bit.
constexpr int kSmallThreads = 1024;

// Workgroup max of v (all lanes receive it).
__device__ __forceinline__ uint32_t small_block_max(uint32_t v) {
  __shared__ uint32_t part[kSmallThreads / 64];
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = part[0];
#pragma unroll
  for (int w = 1; w < kSmallThreads / 64; ++w) m = max(m, part[w]);
  return m;
}

// bf16: x holds nunit 16-element units (2 x 16 bytes each), then ntail < 16
// elements at tail_x.
template <int FMT>
__device__ __forceinline__ void quantize_small_bf16(
    const uint4* __restrict__ x, int64_t nunit, const uint16_t* __restrict__ tail_x,
    uint8_t* __restrict__ tail_y, int ntail, uint4* __restrict__ y, int32_t margin,
    uint32_t* __restrict__ amax, int32_t* __restrict__ bias) {
  const int t = (int)threadIdx.x;
  u16x2 acc = {0, 0};
  for (int64_t i = t; i < 2 * nunit; i += kSmallThreads) acc = vmax_bf16(acc, x[i]);
  uint32_t m = max((uint32_t)acc.x, (uint32_t)acc.y);
  if (t < ntail) m = max(m, (uint32_t)(tail_x[t] & 0x7FFFu));
  const uint32_t a = small_block_max(m) << 16;  // bf16 magnitude widened to fp32 bits
  const int32_t b = bias_from_amax_bits(a, FMT, margin);
  if (t == 0) {
    *amax = a;
    *bias = b;
  }
  const bool hw = kHwConvert<FMT> && b >= kHwBiasMin && b <= kHwBiasMax;
  uint32_t bound2 = 0;
  if constexpr (kHwConvert<FMT>) bound2 = hw_bound2<FMT>(b);
  const float scale = __builtin_ldexpf(1.0f, hw ? -b : 0);
  for (int64_t i = t; i < nunit; i += kSmallThreads) {
    const uint4 lo = x[2 * i], hi = x[2 * i + 1];
    uint4 o;
    if constexpr (kHwConvert<FMT>)
      o = hw ? cast_unit_hw<FMT>(lo, hi, b, bound2, scale) : cast_unit_sw<FMT>(lo, hi, b);
    else
      o = cast_unit_sw<FMT>(lo, hi, b);
    y[i] = o;
  }
  if (t < ntail) tail_y[t] = (uint8_t)fp8_code<FMT>((uint32_t)tail_x[t] << 16, b);
}

template <int FMT>
__global__ __launch_bounds__(kSmallThreads) void quantize_small_bf16_kernel(
    const uint4* __restrict__ x, int64_t nunit, const uint16_t* __restrict__ tail_x,
    uint8_t* __restrict__ tail_y, int ntail, uint4* __restrict__ y, int32_t margin,
    uint32_t* __restrict__ amax, int32_t* __restrict__ bias) {
  quantize_small_bf16<FMT>(x, nunit, tail_x, tail_y, ntail, y, margin, amax, bias);
}

// fp32: x holds nvec groups of 4 elements (16 bytes -> one 4-byte word of
// codes), then ntail < 4 elements at tail_x.
template <int FMT>
__device__ __forceinline__ void quantize_small_f32(
    const uint4* __restrict__ x, int64_t nvec, const uint32_t* __restrict__ tail_x,
    uint8_t* __restrict__ tail_y, int ntail, uint32_t* __restrict__ y, int32_t margin,
    uint32_t* __restrict__ amax, int32_t* __restrict__ bias) {
  const int t = (int)threadIdx.x;
  uint32_t m = 0;
  for (int64_t i = t; i < nvec; i += kSmallThreads) m = vmax_f32(m, x[i]);
  if (t < ntail) m = max(m, tail_x[t] & 0x7FFFFFFFu);
  const uint32_t a = small_block_max(m);
  const int32_t b = bias_from_amax_bits(a, FMT, margin);
  if (t == 0) {
    *amax = a;
    *bias = b;
  }
  const bool hw = kHwConvert<FMT> && b >= kHwBiasMin && b <= kHwBiasMax;
  uint32_t bound = 0;
  if constexpr (kHwConvert<FMT>) bound = hw_bound_f32<FMT>(b);
  const float scale = __builtin_ldexpf(1.0f, hw ? -b : 0);
  for (int64_t i = t; i < nvec; i += kSmallThreads) y[i] = cast4_f32<FMT>(x[i], hw, b, bound, scale);
  if (t < ntail) tail_y[t] = (uint8_t)fp8_code<FMT>(tail_x[t], b);
}

template <int FMT>
__global__ __launch_bounds__(kSmallThreads) void quantize_small_f32_kernel(
    const uint4* __restrict__ x, int64_t nvec, const uint32_t* __restrict__ tail_x,
    uint8_t* __restrict__ tail_y, int ntail, uint32_t* __restrict__ y, int32_t margin,
    uint32_t* __restrict__ amax, int32_t* __restrict__ bias) {
  quantize_small_f32<FMT>(x, nvec, tail_x, tail_y, ntail, y, margin, amax, bias);
}

// ---------------------------------------------------------------- several tensors in few launches
// Small tensors (at most the one-workgroup quantisation's size) are quantised
// by one workgroup each, kMultiMax of them per launch.  The others: up to
// kMultiMax tensors in three launches in all: one
// clears every amax word, one reduces every tensor's amax (each tensor has its
// own run of blocks, sized as the single-tensor amax would size its grid),
// one casts every tensor (each block derives its tensor's bias from the amax
// word, block 0 of each tensor stores it).  Every tensor's amax, bias and
// codes are those of fp8_quantize on it alone, bit for bit: the amax is an
// order-independent integer max, and each cast block does what the
// single-tensor cast does for its part of the tensor.
constexpr int kMultiMax = 32;

struct MultiTensor {
  const void* x;
  uint8_t* y;
  uint32_t* amax;
  int32_t* bias;
  int64_t n;
  int32_t dtype, fmt, margin;
  int32_t amax_first, amax_blocks;  // this tensor's blocks in the amax launch
  int32_t cast_first, cast_blocks;  // and in the cast launch
};

struct MultiArgs {
  int32_t count;
  MultiTensor t[kMultiMax];
};

// The entry of the block's tensor: the last whose first block is at most
// blockIdx.x (entries are in launch order).  Read through the kernel-argument
// pointer so that the wave-uniform index stays a scalar load.
__device__ __forceinline__ const __attribute__((address_space(4))) MultiTensor* multi_entry(bool cast) {
  const auto* a = (const __attribute__((address_space(4))) MultiArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const int b = (int)blockIdx.x;
  int i = 0;
  while (i + 1 < a->count && (cast ? a->t[i + 1].cast_first : a->t[i + 1].amax_first) <= b) ++i;
  return &a->t[i];
}

__global__ void multi_clear_kernel(MultiArgs a) {
  const auto* ka = (const __attribute__((address_space(4))) MultiArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  if ((int)threadIdx.x < ka->count) *ka->t[threadIdx.x].amax = 0u;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void multi_amax_kernel(MultiArgs a) {
  const auto* e = multi_entry(false);
  const int64_t blk = (int64_t)blockIdx.x - e->amax_first, nblk = e->amax_blocks;
  const int64_t n = e->n;
  uint32_t m;
  if (e->dtype == FP8_IN_BF16) {
    const int64_t nvec = n / 8;
    const uint16_t* tail = static_cast<const uint16_t*>(e->x) + nvec * 8;
    m = amax_bf16_body<NT>(static_cast<const uint4*>(e->x), nvec, tail, (int)(n - nvec * 8), blk, nblk);
  } else {
    const int64_t nvec = n / 4;
    const uint32_t* tail = static_cast<const uint32_t*>(e->x) + nvec * 4;
    m = amax_f32_body<NT>(static_cast<const uint4*>(e->x), nvec, tail, (int)(n - nvec * 4), blk, nblk);
  }
  block_max_to(m, e->amax);
}

template <int FMT, bool NT>
__device__ __forceinline__ void multi_cast_one(const __attribute__((address_space(4))) MultiTensor* e,
                                               int64_t blk, int64_t nblk) {
  const BiasArg bias{nullptr, e->amax, e->bias, e->margin};
  const int64_t n = e->n;
  if (e->dtype == FP8_IN_BF16) {
    const int64_t nunit = n / 16;
    cast_bf16_whole<FMT, NT, false>(static_cast<const uint4*>(e->x), nunit, bias, reinterpret_cast<uint4*>(e->y),
                                    static_cast<const uint16_t*>(e->x) + nunit * 16, e->y + nunit * 16,
                                    (int)(n - nunit * 16), blk, nblk);
  } else {
    const int64_t nchunk = n / kF32Chunk;
    cast_f32_whole<FMT, NT, false>(static_cast<const uint4*>(e->x), nchunk, bias,
                                   reinterpret_cast<uint32_t*>(e->y),
                                   static_cast<const uint32_t*>(e->x) + nchunk * kF32Chunk,
                                   e->y + nchunk * kF32Chunk, (int)(n - nchunk * kF32Chunk), blk, nblk);
  }
}

// Small tensors (at most the one-workgroup quantisation's size): workgroup b
// quantises tensor b whole, as fp8_quantize's one-workgroup path does.
template <int FMT>
__device__ __forceinline__ void multi_small_one(const __attribute__((address_space(4))) MultiTensor* e) {
  const int64_t n = e->n;
  if (e->dtype == FP8_IN_BF16) {
    const int64_t nunit = n / 16;
    quantize_small_bf16<FMT>(static_cast<const uint4*>(e->x), nunit,
                             static_cast<const uint16_t*>(e->x) + nunit * 16, e->y + nunit * 16,
                             (int)(n - nunit * 16), reinterpret_cast<uint4*>(e->y), e->margin, e->amax,
                             e->bias);
  } else {
    const int64_t nvec = n / 4;
    quantize_small_f32<FMT>(static_cast<const uint4*>(e->x), nvec, static_cast<const uint32_t*>(e->x) + nvec * 4,
                            e->y + nvec * 4, (int)(n - nvec * 4), reinterpret_cast<uint32_t*>(e->y), e->margin,
                            e->amax, e->bias);
  }
}

__global__ __launch_bounds__(kSmallThreads) void multi_small_kernel(MultiArgs a) {
  const auto* ka = (const __attribute__((address_space(4))) MultiArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const auto* e = &ka->t[blockIdx.x];
  switch (e->fmt) {
    case FP8_E4M3: multi_small_one<FP8_E4M3>(e); break;
    case FP8_E5M2: multi_small_one<FP8_E5M2>(e); break;
    default: multi_small_one<FP8_E3M4>(e); break;
  }
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void multi_cast_kernel(MultiArgs a) {
  const auto* e = multi_entry(true);
  const int64_t blk = (int64_t)blockIdx.x - e->cast_first, nblk = e->cast_blocks;
  switch (e->fmt) {
    case FP8_E4M3: multi_cast_one<FP8_E4M3, NT>(e, blk, nblk); break;
    case FP8_E5M2: multi_cast_one<FP8_E5M2, NT>(e, blk, nblk); break;
    default: multi_cast_one<FP8_E3M4, NT>(e, blk, nblk); break;
  }
}

}  // namespace

// Load hint of amax and cast: non-temporal unless the environment variable
// says "cached" (tuning).
static bool streams(const char* var) {
  const char* h = std::getenv(var);
  return !(h && std::strcmp(h, "cached") == 0);
}

hipError_t launch_amax(const void* x, int dtype, int64_t n, float* amax, hipStream_t stream) {
  uint32_t* out = reinterpret_cast<uint32_t*>(amax);
  hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(1), 0, stream, out);
  if (n > 0) {
    const bool nt = streams("FP8LIN_AMAX_HINT");
    if (dtype == FP8_IN_BF16) {
      const int64_t nvec = n / 8;
      const int ntail = (int)(n - nvec * 8);
      const uint16_t* tail = static_cast<const uint16_t*>(x) + nvec * 8;
      const dim3 grid(stream_blocks(nvec, kAmaxUnroll, kAmaxMaxBlocks));
      const uint4* xv = static_cast<const uint4*>(x);
      if (nt) hipLaunchKernelGGL(amax_bf16_kernel<true>, grid, dim3(kThreads), 0, stream, xv, nvec, tail, ntail, out);
      else hipLaunchKernelGGL(amax_bf16_kernel<false>, grid, dim3(kThreads), 0, stream, xv, nvec, tail, ntail, out);
    } else {
      const int64_t nvec = n / 4;
      const int ntail = (int)(n - nvec * 4);
      const uint32_t* tail = static_cast<const uint32_t*>(x) + nvec * 4;
      const dim3 grid(stream_blocks(nvec, kAmaxUnroll, kAmaxMaxBlocks));
      const uint4* xv = static_cast<const uint4*>(x);
      if (nt) hipLaunchKernelGGL(amax_f32_kernel<true>, grid, dim3(kThreads), 0, stream, xv, nvec, tail, ntail, out);
      else hipLaunchKernelGGL(amax_f32_kernel<false>, grid, dim3(kThreads), 0, stream, xv, nvec, tail, ntail, out);
    }
  }
  return hipGetLastError();
}

hipError_t launch_clear_u32(uint32_t* p, hipStream_t stream) {
  hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(1), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bias(const float* amax, int fmt, int32_t margin, int32_t* bias,
                       hipStream_t stream) {
  hipLaunchKernelGGL(bias_kernel, dim3(1), dim3(1), 0, stream,
                     reinterpret_cast<const uint32_t*>(amax), fmt, margin, bias);
  return hipGetLastError();
}

// Calls fn(format, non-temporal, amax) with each as a std::integral_constant,
// so that one launch statement covers every kernel variant.
template <typename Fn>
void with_cast_variant(int fmt, bool nt, bool amax, Fn&& fn) {
  auto by_amax = [&](auto f, auto n) {
    if (amax) fn(f, n, std::true_type{});
    else fn(f, n, std::false_type{});
  };
  auto by_nt = [&](auto f) {
    if (nt) by_amax(f, std::true_type{});
    else by_amax(f, std::false_type{});
  };
  switch (fmt) {
    case FP8_E4M3: by_nt(std::integral_constant<int, FP8_E4M3>{}); break;
    case FP8_E5M2: by_nt(std::integral_constant<int, FP8_E5M2>{}); break;
    default: by_nt(std::integral_constant<int, FP8_E3M4>{}); break;
  }
}

static hipError_t launch_cast_from(const void* x, int dtype, int64_t n, const BiasArg& bias, int fmt,
                                   uint8_t* y, uint32_t* amax, hipStream_t stream) {
  const bool nt = streams("FP8LIN_CAST_HINT");
  if (amax && n <= 0) {
    if (bias.amax)
      hipLaunchKernelGGL(delayed_empty_kernel, dim3(1), dim3(1), 0, stream, amax, fmt, bias.margin,
                         bias.bias_out);
    else
      hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(1), 0, stream, amax);
    return hipGetLastError();
  }
  if (amax) {
    // the cast with its input's amax: two launches, see cast_part_*_kernel
    if (dtype == FP8_IN_BF16) {
      const int64_t nunit = n / 16;
      const int ntail = (int)(n - nunit * 16);
      const uint16_t* tail_x = static_cast<const uint16_t*>(x) + nunit * 16;
      uint8_t* tail_y = y + nunit * 16;
      const uint4* xv = static_cast<const uint4*>(x);
      uint4* yv = reinterpret_cast<uint4*>(y);
      int64_t first = 0;  // the last block's stretch starts at this unit
      int nwords = 0;
      if (nunit > kPartSmallUnits) {
        const int64_t nb0 = stream_blocks(nunit, kCastUnitsPerLane, kPartMaxBlocksBf16);
        first = nunit - (nb0 + 7) / 8;  // 16 code bytes hold eight 16-bit words
        nwords = stream_blocks(first, kCastUnitsPerLane, kPartMaxBlocksBf16);  // <= nb0
      }
      uint4* stretch = yv + first;
      with_cast_variant(fmt, nt, false, [&](auto f, auto t, auto) {
        constexpr int F = decltype(f)::value;
        constexpr bool T = decltype(t)::value;
        if (nwords > 0)
          hipLaunchKernelGGL((cast_part_bf16_kernel<F, T>), dim3(nwords), dim3(kThreads), 0, stream,
                             xv, first, bias, yv, reinterpret_cast<uint16_t*>(stretch));
        hipLaunchKernelGGL((cast_last_bf16_kernel<F, T>), dim3(1), dim3(kLastThreads), 0, stream,
                           xv + 2 * first, (int)(nunit - first), bias, stretch,
                           reinterpret_cast<const uint32_t*>(stretch), nwords, tail_x, tail_y, ntail,
                           amax);
      });
    } else {
      const int64_t nchunk = n / kF32Chunk;
      const int nrest = (int)(n - nchunk * kF32Chunk);
      const uint32_t* rest_x = static_cast<const uint32_t*>(x) + nchunk * kF32Chunk;
      uint8_t* rest_y = y + nchunk * kF32Chunk;
      const uint4* xv = static_cast<const uint4*>(x);
      uint32_t* yw = reinterpret_cast<uint32_t*>(y);
      constexpr int64_t kChunksPerBlock = kPartThreadsF32 / 64;  // one per wave
      int64_t first = 0;  // in chunks
      int nwords = 0;
      if (nchunk > kPartSmallChunks) {
        const int64_t nb0 = stream_blocks_of(nchunk, 1, kPartMaxBlocksF32, kChunksPerBlock);
        first = nchunk - (nb0 + kF32Chunk / 4 - 1) / (kF32Chunk / 4);  // a chunk's codes hold 256 words
        nwords = stream_blocks_of(first, 1, kPartMaxBlocksF32, kChunksPerBlock);  // <= nb0
      }
      uint32_t* stretch = yw + first * (kF32Chunk / 4);
      with_cast_variant(fmt, nt, false, [&](auto f, auto t, auto) {
        constexpr int F = decltype(f)::value;
        constexpr bool T = decltype(t)::value;
        if (nwords > 0)
          hipLaunchKernelGGL((cast_part_f32_kernel<F, T>), dim3(nwords), dim3(kPartThreadsF32), 0,
                             stream, xv, first, bias, yw, stretch);
        hipLaunchKernelGGL((cast_last_f32_kernel<F, T>), dim3(1), dim3(kLastThreads), 0, stream,
                           xv + first * (kF32Chunk / 4), nchunk - first, bias, stretch, stretch, nwords,
                           rest_x, rest_y, nrest, amax);
      });
    }
    return hipGetLastError();
  }
  if (n <= 0) return hipGetLastError();
  if (dtype == FP8_IN_BF16) {
    // 16-element units, one per lane; the last n % 16 elements by block 0
    const int64_t nunit = n / 16;
    const int ntail = (int)(n - nunit * 16);
    uint8_t* tail_y = y + nunit * 16;
    uint4* yv = reinterpret_cast<uint4*>(y);
    const uint16_t* tail_x = static_cast<const uint16_t*>(x) + nunit * 16;
    const uint4* xv = static_cast<const uint4*>(x);
    const dim3 grid(stream_blocks(nunit, kCastUnitsPerLane, kCastMaxBlocks));
    with_cast_variant(fmt, nt, false, [&](auto f, auto t, auto) {
      hipLaunchKernelGGL((cast_bf16_kernel<decltype(f)::value, decltype(t)::value>),
                         grid, dim3(kThreads), 0, stream, xv, nunit, bias, yv, tail_x, tail_y, ntail);
    });
  } else {
    const int64_t nchunk = n / kF32Chunk;
    const int nrest = (int)(n - nchunk * kF32Chunk);
    const uint32_t* rest_x = static_cast<const uint32_t*>(x) + nchunk * kF32Chunk;
    uint8_t* rest_y = y + nchunk * kF32Chunk;
    uint32_t* yw = reinterpret_cast<uint32_t*>(y);
    const uint4* xv = static_cast<const uint4*>(x);
    // one chunk per wave, four waves per block, at least one block (the rest)
    const int64_t per_block = kThreads / 64;
    const int64_t want = (nchunk + per_block - 1) / per_block;
    const dim3 grid((uint32_t)(want < 1 ? 1 : (want > kCastMaxBlocks ? kCastMaxBlocks : want)));
    with_cast_variant(fmt, nt, false, [&](auto f, auto t, auto) {
      hipLaunchKernelGGL((cast_f32_kernel<decltype(f)::value, decltype(t)::value>),
                         grid, dim3(kThreads), 0, stream, xv, nchunk, bias, yw, rest_x, rest_y, nrest);
    });
  }
  return hipGetLastError();
}

hipError_t launch_quantize_delayed(const void* x, int dtype, int64_t n, int fmt, int32_t margin,
                                   uint8_t* y, float* amax, int32_t* bias, hipStream_t stream) {
  uint32_t* a = reinterpret_cast<uint32_t*>(amax);
  return launch_cast_from(x, dtype, n, BiasArg{nullptr, a, bias, margin}, fmt, y, a, stream);
}

hipError_t launch_cast(const void* x, int dtype, int64_t n, const int32_t* bias, int fmt,
                       uint8_t* y, uint32_t* amax, hipStream_t stream) {
  return launch_cast_from(x, dtype, n, BiasArg{bias, nullptr, nullptr, 0}, fmt, y, amax, stream);
}

// Inputs of at most this many bytes are quantised by one workgroup in one
// launch; larger ones by the amax kernels and a cast that derives the bias
// from the amax itself (three launches: clear, amax, cast).  Measured on
// MI355X, calls back to back on one stream: one workgroup 8.4 us per call up
// to 256 KiB of input (bf16 and fp32 alike), 14 us at 512 KiB, against
// 13.3 us for the three launches at any size up to 8 MiB.
// FP8LIN_QUANT_SMALL (elements) overrides the threshold (tuning and tests).
constexpr int64_t kSmallQuantBytes = 256 * 1024;
static int64_t small_quant_max(int dtype) {
  if (const char* v = std::getenv("FP8LIN_QUANT_SMALL")) return std::atoll(v);
  return kSmallQuantBytes / (dtype == FP8_IN_BF16 ? 2 : 4);
}

hipError_t launch_quantize(const void* x, int dtype, int64_t n, int fmt, int32_t margin, uint8_t* y,
                           float* amax, int32_t* bias, hipStream_t stream) {
  uint32_t* a = reinterpret_cast<uint32_t*>(amax);
  if (n == 0 || n <= small_quant_max(dtype)) {  // an empty tensor still writes amax and bias
    const uint4* xv = static_cast<const uint4*>(x);
    if (dtype == FP8_IN_BF16) {
      const int64_t nunit = n / 16;
      const int ntail = (int)(n - nunit * 16);
      const uint16_t* tail_x = static_cast<const uint16_t*>(x) + nunit * 16;
      uint8_t* tail_y = y + nunit * 16;
      uint4* yv = reinterpret_cast<uint4*>(y);
      with_cast_variant(fmt, false, false, [&](auto f, auto, auto) {
        hipLaunchKernelGGL((quantize_small_bf16_kernel<decltype(f)::value>), dim3(1),
                           dim3(kSmallThreads), 0, stream, xv, nunit, tail_x, tail_y, ntail, yv,
                           margin, a, bias);
      });
    } else {
      const int64_t nvec = n / 4;
      const int ntail = (int)(n - nvec * 4);
      const uint32_t* tail_x = static_cast<const uint32_t*>(x) + nvec * 4;
      uint8_t* tail_y = y + nvec * 4;
      uint32_t* yw = reinterpret_cast<uint32_t*>(y);
      with_cast_variant(fmt, false, false, [&](auto f, auto, auto) {
        hipLaunchKernelGGL((quantize_small_f32_kernel<decltype(f)::value>), dim3(1),
                           dim3(kSmallThreads), 0, stream, xv, nvec, tail_x, tail_y, ntail, yw,
                           margin, a, bias);
      });
    }
    return hipGetLastError();
  }
  if (hipError_t e = launch_amax(x, dtype, n, amax, stream)) return e;
  return launch_cast_from(x, dtype, n, BiasArg{nullptr, a, bias, margin}, fmt, y, nullptr, stream);
}

static MultiTensor multi_entry_of(const QuantDesc& q) {
  MultiTensor t{};
  t.x = q.x;
  t.y = q.y;
  t.amax = reinterpret_cast<uint32_t*>(q.amax);
  t.bias = q.bias;
  t.n = q.n;
  t.dtype = q.dtype;
  t.fmt = q.fmt;
  t.margin = q.margin;
  return t;
}

hipError_t launch_quantize_multi(const QuantDesc* d, int count, hipStream_t stream) {
  // small tensors: one workgroup each, all in one launch (per kMultiMax)
  {
    MultiArgs a{};
    for (int i = 0; i < count; ++i) {
      const QuantDesc& q = d[i];
      if (!(q.n == 0 || q.n <= small_quant_max(q.dtype))) continue;
      a.t[a.count++] = multi_entry_of(q);
      if (a.count == kMultiMax || i == count - 1) {
        hipLaunchKernelGGL(multi_small_kernel, dim3(a.count), dim3(kSmallThreads), 0, stream, a);
        a.count = 0;
      }
    }
    if (a.count > 0) hipLaunchKernelGGL(multi_small_kernel, dim3(a.count), dim3(kSmallThreads), 0, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  // the rest: clear, amax and cast launches for kMultiMax tensors at a time
  const bool nt_amax = streams("FP8LIN_AMAX_HINT"), nt_cast = streams("FP8LIN_CAST_HINT");
  int next = 0;
  while (true) {
    MultiArgs a{};
    while (next < count && a.count < kMultiMax) {
      const QuantDesc& q = d[next++];
      if (!(q.n == 0 || q.n <= small_quant_max(q.dtype))) a.t[a.count++] = multi_entry_of(q);
    }
    if (a.count == 0) break;
    int64_t amax_total = 0, cast_total = 0;
    for (int i = 0; i < a.count; ++i) {
      MultiTensor& t = a.t[i];
      const QuantDesc q{t.x, t.n, t.dtype, t.fmt, t.margin, t.y, reinterpret_cast<float*>(t.amax), t.bias};
      // the grids the single-tensor amax and cast would launch
      const bool bf = q.dtype == FP8_IN_BF16;
      t.amax_blocks = stream_blocks(bf ? q.n / 8 : q.n / 4, kAmaxUnroll, kAmaxMaxBlocks);
      if (bf) {
        t.cast_blocks = stream_blocks(q.n / 16, kCastUnitsPerLane, kCastMaxBlocks);
      } else {
        const int64_t want = (q.n / kF32Chunk + (kThreads / 64) - 1) / (kThreads / 64);
        t.cast_blocks = (int)(want < 1 ? 1 : (want > kCastMaxBlocks ? kCastMaxBlocks : want));
      }
      t.amax_first = (int32_t)amax_total;
      t.cast_first = (int32_t)cast_total;
      amax_total += t.amax_blocks;
      cast_total += t.cast_blocks;
    }
    hipLaunchKernelGGL(multi_clear_kernel, dim3(1), dim3(64), 0, stream, a);
    if (nt_amax) hipLaunchKernelGGL(multi_amax_kernel<true>, dim3((uint32_t)amax_total), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(multi_amax_kernel<false>, dim3((uint32_t)amax_total), dim3(kThreads), 0, stream, a);
    if (nt_cast) hipLaunchKernelGGL(multi_cast_kernel<true>, dim3((uint32_t)cast_total), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(multi_cast_kernel<false>, dim3((uint32_t)cast_total), dim3(kThreads), 0, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

}  // namespace fp8lin
