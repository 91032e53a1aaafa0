/*
 * A C client of libfp8lin: no Python, only include/fp8lin.h, the shared
 * library and the HIP runtime's C API (for device memory and a stream).
 *
 *   abi_client checks        argument checks and status strings (no device)
 *   abi_client run DIR N     quantise a seeded bf16 vector of N elements to
 *                            E4M3, multiply a 64 x 128 product of it with a
 *                            seeded E4M3 weight, add the product onto a
 *                            copy of it (fp8_scaled_gemm_accumulate), and
 *                            write the amax, bias, codes and both outputs to
 *                            DIR as raw files
 * Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8lin.h"

/* The few HIP runtime entry points used, declared here with C linkage. */
typedef int hipError_t;
typedef void* hipStream_t;
extern hipError_t hipMalloc(void** p, size_t n);
extern hipError_t hipFree(void* p);
extern hipError_t hipMemcpy(void* dst, const void* src, size_t n, int kind);
extern hipError_t hipStreamCreate(hipStream_t* s);
extern hipError_t hipStreamSynchronize(hipStream_t s);
extern hipError_t hipStreamDestroy(hipStream_t s);
#define H2D 1
#define D2H 2
#define D2D 3

static int expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d\n", what, got, fp8_status_string(got), want);
    return 1;
  }
  return 0;
}

static int checks(void) {
  int bad = 0;
  void* p = (void*)(uintptr_t)64; /* aligned, never dereferenced: every call below fails its checks */
  bad += expect("amax n<0", fp8_amax(p, FP8_IN_BF16, -1, (float*)p, NULL), FP8_ERR_SIZE);
  bad += expect("amax dtype", fp8_amax(p, (fp8_dtype_t)9, 8, (float*)p, NULL), FP8_ERR_DTYPE);
  bad += expect("bias format", fp8_compute_bias((float*)p, (fp8_format_t)7, 0, (int32_t*)p, NULL), FP8_ERR_FORMAT);
  bad += expect("bias margin", fp8_compute_bias((float*)p, FP8_E4M3, FP8_MAX_MARGIN + 1, (int32_t*)p, NULL), FP8_ERR_MARGIN);
  bad += expect("cast null", fp8_scale_cast(p, FP8_IN_FP32, 4, NULL, FP8_E5M2, (uint8_t*)p, NULL), FP8_ERR_NULL);
  bad += expect("gemm E3M4", fp8_scaled_gemm_fwd((uint8_t*)p, FP8_E3M4, (int32_t*)p, (uint8_t*)p, FP8_E4M3, (int32_t*)p, 8, 8, 8, (float*)p, NULL), FP8_ERR_FORMAT);
  bad += expect("gemm op", fp8_scaled_gemm((fp8_gemm_op_t)5, FP8_GEMM_EXACT, (uint8_t*)p, FP8_E4M3, (int32_t*)p, (uint8_t*)p, FP8_E4M3, (int32_t*)p, 8, 8, 8, (float*)p, NULL), FP8_ERR_OP);
  bad += expect("accumulate null", fp8_scaled_gemm_accumulate(FP8_GEMM_WGRAD, FP8_GEMM_EXACT, (uint8_t*)p, FP8_E5M2, (int32_t*)p, (uint8_t*)p, FP8_E4M3, (int32_t*)p, 8, 8, 8, NULL, NULL), FP8_ERR_NULL);
  bad += expect("swiglu size", fp8_swiglu_fwd((float*)p, -2, 4, (uint16_t*)p, NULL, NULL), FP8_ERR_SIZE);
  bad += expect("workspace op", (int)fp8_scaled_gemm_workspace_bytes((fp8_gemm_op_t)7, 8, 8, 64), FP8_ERR_OP);
  if (fp8_scaled_gemm_workspace_bytes(FP8_GEMM_FWD, 128, 8192, 8192) != 4LL * 128 * 8192 * 4) bad++;
  bad += expect("ws too small", fp8_scaled_gemm_ws(FP8_GEMM_FWD, FP8_GEMM_EXACT, (uint8_t*)p, FP8_E4M3, (int32_t*)p, (uint8_t*)p, FP8_E4M3, (int32_t*)p, 128, 8192, 8192, (float*)p, p, 16, NULL), FP8_ERR_SIZE);
  bad += expect("quantize margin", fp8_quantize(p, FP8_IN_BF16, 8, FP8_E4M3, -FP8_MAX_MARGIN - 1, (uint8_t*)p, (float*)p, (int32_t*)p, NULL), FP8_ERR_MARGIN);
  if (strlen(fp8_status_string(FP8_ERR_ALIGN)) == 0) bad++;
  return bad;
}

/* splitmix64: the seeded inputs */
static uint64_t sm_state = 12345;
static uint64_t next_u64(void) {
  uint64_t z = (sm_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static int write_file(const char* dir, const char* name, const void* data, size_t n) {
  char path[1024];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  size_t w = fwrite(data, 1, n, f);
  fclose(f);
  return w != n;
}

#define TRY(call)                                                                      \
  do {                                                                                 \
    int s_ = (call);                                                                   \
    if (s_ != 0) {                                                                     \
      fprintf(stderr, "%s failed: %d (%s)\n", #call, s_, fp8_status_string(s_));      \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)

static int run(const char* dir, int64_t n) {
  const int64_t M = 64, K = 128, N = 48; /* X8 = the first M*K codes, as M x K */
  if (n < M * K) return 2;
  uint16_t* x = malloc((size_t)n * 2);
  uint8_t* w = malloc((size_t)(N * K));
  for (int64_t i = 0; i < n; ++i) {
    /* bf16 with a random sign, exponent 118..133 and fraction */
    uint64_t r = next_u64();
    x[i] = (uint16_t)(((r & 1) << 15) | ((118 + (r >> 1) % 16) << 7) | ((r >> 8) & 0x7F));
  }
  for (int64_t i = 0; i < N * K; ++i) {
    uint8_t c = (uint8_t)(next_u64() & 0xFF);
    if ((c & 0x7F) == 0x7F) c &= 0xF0; /* no NaN codes */
    w[i] = c;
  }
  hipStream_t st;
  void *dx, *dy, *damax, *dbias, *dw, *dbw, *dout;
  if (hipStreamCreate(&st)) return 3;
  if (hipMalloc(&dx, (size_t)n * 2) || hipMalloc(&dy, (size_t)n) || hipMalloc(&damax, 4) ||
      hipMalloc(&dbias, 4) || hipMalloc(&dw, (size_t)(N * K)) || hipMalloc(&dbw, 4) ||
      hipMalloc(&dout, (size_t)(M * N) * 4))
    return 3;
  const int32_t bw = 3;
  if (hipMemcpy(dx, x, (size_t)n * 2, H2D) || hipMemcpy(dw, w, (size_t)(N * K), H2D) ||
      hipMemcpy(dbw, &bw, 4, H2D))
    return 3;
  TRY(fp8_amax(dx, FP8_IN_BF16, n, (float*)damax, st));
  TRY(fp8_compute_bias((const float*)damax, FP8_E4M3, 0, (int32_t*)dbias, st));
  TRY(fp8_scale_cast(dx, FP8_IN_BF16, n, (const int32_t*)dbias, FP8_E4M3, (uint8_t*)dy, st));
  TRY(fp8_scaled_gemm_fwd((const uint8_t*)dy, FP8_E4M3, (const int32_t*)dbias, (const uint8_t*)dw,
                          FP8_E4M3, (const int32_t*)dbw, M, N, K, (float*)dout, st));
  /* the product added onto a copy of itself: twice the product */
  void* dacc;
  if (hipMalloc(&dacc, (size_t)(M * N) * 4) || hipStreamSynchronize(st) ||
      hipMemcpy(dacc, dout, (size_t)(M * N) * 4, D2D))
    return 3;
  TRY(fp8_scaled_gemm_accumulate(FP8_GEMM_FWD, FP8_GEMM_EXACT, (const uint8_t*)dy, FP8_E4M3, (const int32_t*)dbias,
                                 (const uint8_t*)dw, FP8_E4M3, (const int32_t*)dbw, M, N, K, (float*)dacc, st));
  /* the same quantisation in one call, into separate buffers */
  void *dy1, *damax1, *dbias1;
  if (hipMalloc(&dy1, (size_t)n) || hipMalloc(&damax1, 4) || hipMalloc(&dbias1, 4)) return 3;
  TRY(fp8_quantize(dx, FP8_IN_BF16, n, FP8_E4M3, 0, (uint8_t*)dy1, (float*)damax1, (int32_t*)dbias1, st));
  if (hipStreamSynchronize(st)) return 4;
  float amax, amax1;
  int32_t bias, bias1;
  uint8_t* codes = malloc((size_t)n);
  uint8_t* codes1 = malloc((size_t)n);
  if (hipMemcpy(&amax1, damax1, 4, D2H) || hipMemcpy(&bias1, dbias1, 4, D2H) ||
      hipMemcpy(codes1, dy1, (size_t)n, D2H))
    return 4;
  float* out = malloc((size_t)(M * N) * 4);
  float* out2 = malloc((size_t)(M * N) * 4);
  if (hipMemcpy(&amax, damax, 4, D2H) || hipMemcpy(&bias, dbias, 4, D2H) ||
      hipMemcpy(codes, dy, (size_t)n, D2H) || hipMemcpy(out, dout, (size_t)(M * N) * 4, D2H) ||
      hipMemcpy(out2, dacc, (size_t)(M * N) * 4, D2H))
    return 4;
  if (memcmp(&amax, &amax1, 4) != 0 || bias != bias1 || memcmp(codes, codes1, (size_t)n) != 0) {
    fprintf(stderr, "fp8_quantize differs from amax -> compute_bias -> scale_cast\n");
    return 6;
  }
  int bad = write_file(dir, "x.bf16", x, (size_t)n * 2) + write_file(dir, "w.e4m3", w, (size_t)(N * K)) +
            write_file(dir, "amax.f32", &amax, 4) + write_file(dir, "bias.i32", &bias, 4) +
            write_file(dir, "codes.u8", codes, (size_t)n) +
            write_file(dir, "y.f32", out, (size_t)(M * N) * 4) +
            write_file(dir, "y2.f32", out2, (size_t)(M * N) * 4);
  hipFree(dx); hipFree(dy); hipFree(damax); hipFree(dbias); hipFree(dw); hipFree(dbw); hipFree(dout);
  hipFree(dacc);
  hipFree(dy1); hipFree(damax1); hipFree(dbias1);
  hipStreamDestroy(st);
  free(x); free(w); free(codes); free(codes1); free(out); free(out2);
  return bad ? 5 : 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "checks") == 0) return checks();
  if (argc >= 4 && strcmp(argv[1], "run") == 0) return run(argv[2], atoll(argv[3]));
  fprintf(stderr, "usage: abi_client checks | run DIR N\n");
  return 2;
}
