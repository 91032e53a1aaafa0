// The gated activation between the two products of a chained FP8 MLP (Llama 2's
// SwiGLU; the pages train Llama 2 models, "Training and inference of large
// language models using 8-bit floating point", review page, "Main findings"),
// forward and backward, each folding the amax of the tensor it writes, which is
// the next quantisation's input ("Proposed method", bullet 1).
//
//   h  [rows x 2f] fp32, row t = [g_t | u_t]   (the fused gate-up product)
//   forward   a[t][j]      = silu(g) * u                        bf16
//   backward  dh[t][j]     = da * u * sigmoid(g) * (1 + g * (1 - sigmoid(g)))
//             dh[t][f + j] = da * silu(g)                       bf16
//
// HBM-bound elementwise work: 8 bytes read and 2 written per forward output,
// 12 read and 4 written per backward output pair.  Each block takes a slice of
// one row, so the gate and up halves are two contiguous 16-byte streams; a
// lane loads 4 units of 4 elements (streaming loads: h and da are read once)
// before any arithmetic.  The amax is reduced over the block in LDS and folded
// with one atomic per block: with one atomic per wave, the waves' atomics on
// the one address cost more than the kernel's own traffic (measured on
// MI355X over a 4096 x 11008 output: 163 us with one unit per lane and an
// atomic per wave, 72 us without the fold).
#include "internal.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerLane = 4;  // units (of V elements) per lane per block
constexpr int64_t kUnitsPerBlock = (int64_t)kThreads * kUnitsPerLane;

// sigmoid(g) and 1 - sigmoid(g) from e = exp(-|g|): e / (1 + e) and 1 / (1 + e),
// so neither is formed by a subtraction and a very negative g gives a tiny
// (possibly subnormal) sigmoid rather than an overflowed exp.  exp keeps
// subnormal results; 1 + e lies in [1, 2], where the hardware reciprocal
// (1 ulp) needs none of a division's range handling.
__device__ __forceinline__ void sigmoid_pair(float g, float& s, float& sc) {
  const bool neg = g < 0.0f;
  const float e = expf(neg ? g : -g);
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  const float er = e * r;
  s = neg ? er : r;
  sc = neg ? r : er;
}

// fp32 -> bf16 bits, round to nearest even (overflow to inf); NaN stays NaN.
__device__ __forceinline__ uint32_t bf16_bits(float v) {
  const uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x40u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) loads: each input is read once.
template <int V>
__device__ __forceinline__ void load_f32(const float* p, float (&v)[V]) {
  if constexpr (V == 4) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    v[0] = t[0];
    v[1] = t[1];
    v[2] = t[2];
    v[3] = t[3];
  } else {
    v[0] = __builtin_nontemporal_load(p);
  }
}

template <int V>
__device__ __forceinline__ void store_bf16(uint16_t* p, const uint32_t (&w)[V]) {
  if constexpr (V == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
  } else {
    *p = (uint16_t)w[0];
  }
}

// Largest bf16 magnitude of the block (as fp32 bits) into *amax: wave
// shuffles, the four wave maxima through LDS, one atomic per block, skipped
// when the stored value is already at least as large.  Called by every lane.
__device__ __forceinline__ void fold_amax(uint32_t m, uint32_t* amax) {
  __shared__ uint32_t wave_max[kThreads / 64];
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) m = max(m, wave_max[w]);
    if (m > __hip_atomic_load(amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(amax, m);
  }
}

// Block b covers units [part * kUnitsPerBlock, (part + 1) * kUnitsPerBlock) of
// row b / bpr; a unit is V consecutive columns (V = 4 when f % 4 == 0).
template <int V>
__global__ __launch_bounds__(kThreads) void swiglu_fwd_kernel(const float* __restrict__ h,
                                                              int64_t f, int64_t upr, int bpr,
                                                              uint16_t* __restrict__ a,
                                                              uint32_t* __restrict__ amax) {
  const int64_t row = blockIdx.x / bpr;
  const int64_t j0 = (int64_t)(blockIdx.x - row * bpr) * kUnitsPerBlock + threadIdx.x;
  const float* hg = h + row * 2 * f;
  const float* hu = hg + f;
  uint16_t* ar = a + row * f;
  float g[kUnitsPerLane][V], u[kUnitsPerLane][V];
#pragma unroll
  for (int k = 0; k < kUnitsPerLane; ++k) {
    const int64_t j = j0 + k * kThreads;
    if (j < upr) {
      load_f32<V>(hg + j * V, g[k]);
      load_f32<V>(hu + j * V, u[k]);
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < kUnitsPerLane; ++k) {
    const int64_t j = j0 + k * kThreads;
    if (j < upr) {
      uint32_t w[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float s, sc;
        sigmoid_pair(g[k][v], s, sc);
        w[v] = bf16_bits(g[k][v] * s * u[k][v]);
        m = max(m, (w[v] & 0x7FFFu) << 16);
      }
      store_bf16<V>(ar + j * V, w);
    }
  }
  if (amax) fold_amax(m, amax);
}

template <int V>
__global__ __launch_bounds__(kThreads) void swiglu_bwd_kernel(const float* __restrict__ h,
                                                              const float* __restrict__ da,
                                                              int64_t f, int64_t upr, int bpr,
                                                              uint16_t* __restrict__ dh,
                                                              uint32_t* __restrict__ amax) {
  const int64_t row = blockIdx.x / bpr;
  const int64_t j0 = (int64_t)(blockIdx.x - row * bpr) * kUnitsPerBlock + threadIdx.x;
  const float* hg = h + row * 2 * f;
  const float* hu = hg + f;
  const float* dar = da + row * f;
  uint16_t* dg_out = dh + row * 2 * f;
  uint16_t* du_out = dg_out + f;
  float g[kUnitsPerLane][V], u[kUnitsPerLane][V], d[kUnitsPerLane][V];
#pragma unroll
  for (int k = 0; k < kUnitsPerLane; ++k) {
    const int64_t j = j0 + k * kThreads;
    if (j < upr) {
      load_f32<V>(hg + j * V, g[k]);
      load_f32<V>(hu + j * V, u[k]);
      load_f32<V>(dar + j * V, d[k]);
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < kUnitsPerLane; ++k) {
    const int64_t j = j0 + k * kThreads;
    if (j < upr) {
      uint32_t wg[V], wu[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float gv = g[k][v];
        float s, sc;
        sigmoid_pair(gv, s, sc);
        wg[v] = bf16_bits(d[k][v] * u[k][v] * (s * (1.0f + gv * sc)));
        wu[v] = bf16_bits(d[k][v] * (gv * s));
        m = max(m, max((wg[v] & 0x7FFFu) << 16, (wu[v] & 0x7FFFu) << 16));
      }
      store_bf16<V>(dg_out + j * V, wg);
      store_bf16<V>(du_out + j * V, wu);
    }
  }
  if (amax) fold_amax(m, amax);
}

__global__ void clear_kernel(uint32_t* p) { *p = 0u; }

struct Grid {
  int64_t upr;  // units per row
  int bpr;      // blocks per row
  int64_t blocks;
  bool vec;
};

Grid grid_of(int64_t rows, int64_t f) {
  Grid g;
  g.vec = (f % 4) == 0;
  g.upr = g.vec ? f / 4 : f;
  g.bpr = (int)((g.upr + kUnitsPerBlock - 1) / kUnitsPerBlock);
  g.blocks = rows * g.bpr;
  return g;
}

}  // namespace

int64_t swiglu_blocks(int64_t rows, int64_t f) { return grid_of(rows, f).blocks; }

hipError_t launch_swiglu_fwd(const float* h, int64_t rows, int64_t f, uint16_t* a, uint32_t* amax,
                             hipStream_t stream) {
  if (amax) hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, stream, amax);
  if (rows > 0 && f > 0) {
    const Grid g = grid_of(rows, f);
    if (g.vec)
      hipLaunchKernelGGL(swiglu_fwd_kernel<4>, dim3((uint32_t)g.blocks), dim3(kThreads), 0, stream,
                         h, f, g.upr, g.bpr, a, amax);
    else
      hipLaunchKernelGGL(swiglu_fwd_kernel<1>, dim3((uint32_t)g.blocks), dim3(kThreads), 0, stream,
                         h, f, g.upr, g.bpr, a, amax);
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* h, const float* da, int64_t rows, int64_t f, uint16_t* dh,
                             uint32_t* amax, hipStream_t stream) {
  if (amax) hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, stream, amax);
  if (rows > 0 && f > 0) {
    const Grid g = grid_of(rows, f);
    if (g.vec)
      hipLaunchKernelGGL(swiglu_bwd_kernel<4>, dim3((uint32_t)g.blocks), dim3(kThreads), 0, stream,
                         h, da, f, g.upr, g.bpr, dh, amax);
    else
      hipLaunchKernelGGL(swiglu_bwd_kernel<1>, dim3((uint32_t)g.blocks), dim3(kThreads), 0, stream,
                         h, da, f, g.upr, g.bpr, dh, amax);
  }
  return hipGetLastError();
}

}  // namespace fp8lin
