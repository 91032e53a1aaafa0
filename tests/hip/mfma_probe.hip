// Test-only probes of single MFMA instructions on gfx950: one wave runs one
// instruction on register images the host supplies, and returns the
// accumulator registers.  Used to measure how each instruction sums its
// products (how far below the largest product a term still counts), which
// decides what arithmetic the FP8 products can use under an elementwise
// 1e-5 * sum |a||b| tolerance.  Not part of libfp8lin.
//
// Register images (per lane, 32 bytes each operand; an instruction reads the
// first 8, 16 or 32): lane l of the host buffers is lane l of the wave.
// Output: 16 floats per lane (16x16 instructions fill the first 4).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

enum Kind {
  kF8F6F4_32x32x64 = 0,   // v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales
  kF8F6F4_16x16x128 = 1,  // v_mfma_scale_f32_16x16x128_f8f6f4, unit block scales
  kFp8_32x32x16 = 2,      // v_mfma_f32_32x32x16_{fp8,bf8}_{fp8,bf8}
  kF16_32x32x16 = 3,      // v_mfma_f32_32x32x16_f16
  kBf16_32x32x16 = 4,     // v_mfma_f32_32x32x16_bf16
};

template <int FA, int FB>
__global__ void f8f6f4_32(const v8i* a, const v8i* b, v16f* out) {
  const int l = threadIdx.x;
  v16f c = {};
  out[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], c, FA, FB, 0, 127, 0, 127);
}

template <int FA, int FB>
__global__ void f8f6f4_16(const v8i* a, const v8i* b, v16f* out) {
  const int l = threadIdx.x;
  v4f c = {};
  const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[l], b[l], c, FA, FB, 0, 127, 0, 127);
  v16f o = {};
  for (int i = 0; i < 4; ++i) o[i] = r[i];
  out[l] = o;
}

template <int FA, int FB>
__global__ void fp8_32(const v8i* a, const v8i* b, v16f* out) {
  const int l = threadIdx.x;
  const long x = ((long)(uint32_t)a[l][1] << 32) | (uint32_t)a[l][0];
  const long y = ((long)(uint32_t)b[l][1] << 32) | (uint32_t)b[l][0];
  v16f c = {};
  if constexpr (FA == 0 && FB == 0) out[l] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(x, y, c, 0, 0, 0);
  else if constexpr (FA == 1 && FB == 0) out[l] = __builtin_amdgcn_mfma_f32_32x32x16_bf8_fp8(x, y, c, 0, 0, 0);
  else if constexpr (FA == 0 && FB == 1) out[l] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_bf8(x, y, c, 0, 0, 0);
  else out[l] = __builtin_amdgcn_mfma_f32_32x32x16_bf8_bf8(x, y, c, 0, 0, 0);
}

__global__ void f16_32(const v8i* a, const v8i* b, v16f* out) {
  const int l = threadIdx.x;
  const v8h x = __builtin_bit_cast(v8h, (int __attribute__((ext_vector_type(4)))){a[l][0], a[l][1], a[l][2], a[l][3]});
  const v8h y = __builtin_bit_cast(v8h, (int __attribute__((ext_vector_type(4)))){b[l][0], b[l][1], b[l][2], b[l][3]});
  v16f c = {};
  out[l] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c, 0, 0, 0);
}

__global__ void bf16_32(const v8i* a, const v8i* b, v16f* out) {
  const int l = threadIdx.x;
  const v8bf x = __builtin_bit_cast(v8bf, (int __attribute__((ext_vector_type(4)))){a[l][0], a[l][1], a[l][2], a[l][3]});
  const v8bf y = __builtin_bit_cast(v8bf, (int __attribute__((ext_vector_type(4)))){b[l][0], b[l][1], b[l][2], b[l][3]});
  v16f c = {};
  out[l] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
}

#define PROBE_FMT_SWITCH(KERNEL)                                                              \
  if (fa == 0 && fb == 0) hipLaunchKernelGGL((KERNEL<0, 0>), dim3(1), dim3(64), 0, 0, a, b, o); \
  else if (fa == 1 && fb == 0) hipLaunchKernelGGL((KERNEL<1, 0>), dim3(1), dim3(64), 0, 0, a, b, o); \
  else if (fa == 0 && fb == 1) hipLaunchKernelGGL((KERNEL<0, 1>), dim3(1), dim3(64), 0, 0, a, b, o); \
  else if (fa == 1 && fb == 1) hipLaunchKernelGGL((KERNEL<1, 1>), dim3(1), dim3(64), 0, 0, a, b, o); \
  else return -2;

}  // namespace

extern "C" {

// One instruction of `kind` on the register images a_img, b_img (host, 64 x 32
// bytes each); writes 64 x 16 floats to out (host).  fa, fb: 0 = E4M3 (fp8),
// 1 = E5M2 (bf8), for the FP8 kinds.  Returns 0, -1 for a HIP error, -2 for
// an unknown kind or format.
int probe_mfma(int kind, int fa, int fb, const void* a_img, const void* b_img, float* out) {
  v8i *a = nullptr, *b = nullptr;
  v16f* o = nullptr;
  int rc = -1;
  if (hipMalloc(&a, 64 * 32) != hipSuccess || hipMalloc(&b, 64 * 32) != hipSuccess ||
      hipMalloc(&o, 64 * 64) != hipSuccess)
    goto done;
  if (hipMemcpy(a, a_img, 64 * 32, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(b, b_img, 64 * 32, hipMemcpyHostToDevice) != hipSuccess)
    goto done;
  switch (kind) {
    case kF8F6F4_32x32x64: PROBE_FMT_SWITCH(f8f6f4_32) break;
    case kF8F6F4_16x16x128: PROBE_FMT_SWITCH(f8f6f4_16) break;
    case kFp8_32x32x16: PROBE_FMT_SWITCH(fp8_32) break;
    case kF16_32x32x16: hipLaunchKernelGGL(f16_32, dim3(1), dim3(64), 0, 0, a, b, o); break;
    case kBf16_32x32x16: hipLaunchKernelGGL(bf16_32, dim3(1), dim3(64), 0, 0, a, b, o); break;
    default: rc = -2; goto done;
  }
  if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) goto done;
  if (hipMemcpy(out, o, 64 * 64, hipMemcpyDeviceToHost) != hipSuccess) goto done;
  rc = 0;
done:
  if (a) (void)hipFree(a);
  if (b) (void)hipFree(b);
  if (o) (void)hipFree(o);
  return rc;
}

}  // extern "C"
