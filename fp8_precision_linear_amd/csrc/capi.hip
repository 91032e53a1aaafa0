// C ABI of libfp8lin: argument checks on the host, then kernel launches on the
// caller's stream.  No allocation, no host synchronisation, no state beyond a
// per-device "is this gfx950" flag and the per-device address of the static
// scratch that fp8_scaled_gemm_noalloc uses.
#include <atomic>
#include <cstring>

#include "internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = something else.
std::atomic<int> g_arch_ok[kMaxDevices];

// The split workspace of fp8_scaled_gemm_noalloc, for callers that cannot
// allocate: one copy per device, held until the process ends.  Host code never
// passes `scratch` itself (on the host it names a stand-in, not device memory):
// it passes the device address hipGetSymbolAddress returns for the current
// device, looked up on the first call on that device and kept in g_scratch.
static __device__ __align__(256) __attribute__((used)) uint8_t scratch[FP8_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }
// amax and bias words: their natural 4-byte alignment (atomics need it)
bool misaligned_word(const void* p) { return ((uintptr_t)p & 3u) != 0; }
// E3M4 has no MFMA operand type: quantisation only.
bool bad_format(int f) { return f != FP8_E4M3 && f != FP8_E5M2 && f != FP8_E3M4; }
bool bad_operand_format(int f) { return f != FP8_E4M3 && f != FP8_E5M2; }
bool bad_dtype(int d) { return d != FP8_IN_BF16 && d != FP8_IN_FP32; }
bool bad_dim(int64_t v) { return v < 0 || v > (int64_t)0x7FFFFFFF; }

// The current device must be a gfx950.  Checked once per device.
int device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8_ERR_DEVICE;
  if (dev >= kMaxDevices) return FP8_ERR_DEVICE;
  int state = g_arch_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? FP8_OK : FP8_ERR_DEVICE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_HIP; }

// The current device's copy of `scratch` (device_ok() has already checked the
// device index).  Several threads may look it up at once: each gets the same
// address.
int scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8_ERR_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return FP8_OK;
}

// The operands are a_rows x a_cols and b_rows x b_cols, each of those one of
// M, N, K: the products are formed only after the range check.
int gemm_checks(const uint8_t* a, int fa, const int32_t* ba, const uint8_t* b, int fb,
                const int32_t* bb, int64_t M, int64_t N, int64_t K, const float* out,
                int64_t a_rows, int64_t a_cols, int64_t b_rows, int64_t b_cols) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return FP8_ERR_SIZE;
  const int64_t a_elems = a_rows * a_cols, b_elems = b_rows * b_cols;
  // the launch grid (at most one block per 128 x 128 output tile) is 32-bit
  if (((M + 127) / 128) * ((N + 127) / 128) > (int64_t)0x7FFFFFFF) return FP8_ERR_SIZE;
  if (bad_operand_format(fa) || bad_operand_format(fb)) return FP8_ERR_FORMAT;
  if (M == 0 || N == 0) return FP8_OK;
  if (!out || !ba || !bb) return FP8_ERR_NULL;
  if ((a_elems > 0 && !a) || (b_elems > 0 && !b)) return FP8_ERR_NULL;
  if (misaligned(out) || (a && misaligned(a)) || (b && misaligned(b))) return FP8_ERR_ALIGN;
  if (misaligned_word(ba) || misaligned_word(bb)) return FP8_ERR_ALIGN;
  return FP8_OK;
}

// fp8_quantize's argument checks (no device call).
int quantize_checks(const void* x, int dtype, int64_t n, int fmt, int32_t margin, const uint8_t* y,
                    const float* amax, const int32_t* bias) {
  if (n < 0) return FP8_ERR_SIZE;
  if (bad_dtype(dtype)) return FP8_ERR_DTYPE;
  if (bad_format(fmt)) return FP8_ERR_FORMAT;
  if (margin > FP8_MAX_MARGIN || margin < -FP8_MAX_MARGIN) return FP8_ERR_MARGIN;
  if (!amax || !bias || (n > 0 && (!x || !y))) return FP8_ERR_NULL;
  if (misaligned_word(amax) || misaligned_word(bias)) return FP8_ERR_ALIGN;
  if (n > 0 && (misaligned(x) || misaligned(y))) return FP8_ERR_ALIGN;
  return FP8_OK;
}

}  // namespace

extern "C" {

const char* fp8_status_string(int status) {
  switch (status) {
    case FP8_OK: return "ok";
    case FP8_ERR_NULL: return "a required pointer is NULL";
    case FP8_ERR_SIZE: return "a size is negative or too large";
    case FP8_ERR_FORMAT: return "unknown FP8 format";
    case FP8_ERR_DTYPE: return "unknown input dtype";
    case FP8_ERR_ALIGN: return "a pointer is misaligned (16 bytes for tensors, 4 for amax outputs)";
    case FP8_ERR_MARGIN: return "margin out of range";
    case FP8_ERR_DEVICE: return "no gfx950 HIP device is current";
    case FP8_ERR_HIP: return "a HIP launch failed";
    case FP8_ERR_OP: return "unknown product or math selector";
    default: return "unknown status";
  }
}

int fp8_amax(const void* x, fp8_dtype_t dtype, int64_t n, float* amax, void* stream) {
  if (n < 0) return FP8_ERR_SIZE;
  if (bad_dtype(dtype)) return FP8_ERR_DTYPE;
  if (!amax || (n > 0 && !x)) return FP8_ERR_NULL;
  if ((n > 0 && misaligned(x)) || misaligned_word(amax)) return FP8_ERR_ALIGN;
  if (int s = device_ok()) return s;
  return hip_status(fp8lin::launch_amax(x, dtype, n, amax, (hipStream_t)stream));
}

int fp8_compute_bias(const float* amax, fp8_format_t fmt, int32_t margin, int32_t* bias,
                     void* stream) {
  if (bad_format(fmt)) return FP8_ERR_FORMAT;
  if (margin > FP8_MAX_MARGIN || margin < -FP8_MAX_MARGIN) return FP8_ERR_MARGIN;
  if (!amax || !bias) return FP8_ERR_NULL;
  if (misaligned_word(amax) || misaligned_word(bias)) return FP8_ERR_ALIGN;
  if (int s = device_ok()) return s;
  return hip_status(fp8lin::launch_bias(amax, fmt, margin, bias, (hipStream_t)stream));
}

int fp8_scale_cast(const void* x, fp8_dtype_t dtype, int64_t n, const int32_t* bias,
                   fp8_format_t fmt, uint8_t* y, void* stream) {
  if (n < 0) return FP8_ERR_SIZE;
  if (bad_dtype(dtype)) return FP8_ERR_DTYPE;
  if (bad_format(fmt)) return FP8_ERR_FORMAT;
  if (n == 0) return FP8_OK;
  if (!x || !y || !bias) return FP8_ERR_NULL;
  if (misaligned(x) || misaligned(y) || misaligned_word(bias)) return FP8_ERR_ALIGN;
  if (int s = device_ok()) return s;
  return hip_status(fp8lin::launch_cast(x, dtype, n, bias, fmt, y, nullptr, (hipStream_t)stream));
}

int fp8_quantize(const void* x, fp8_dtype_t dtype, int64_t n, fp8_format_t fmt, int32_t margin,
                 uint8_t* y, float* amax, int32_t* bias, void* stream) {
  if (int s = quantize_checks(x, dtype, n, fmt, margin, y, amax, bias)) return s;
  if (int s = device_ok()) return s;
  return hip_status(fp8lin::launch_quantize(x, dtype, n, fmt, margin, y, amax, bias,
                                            (hipStream_t)stream));
}

int fp8_quantize_multi(const fp8_quant_desc_t* descs, int32_t count, void* stream) {
  if (count < 0) return FP8_ERR_SIZE;
  if (count == 0) return FP8_OK;
  if (!descs) return FP8_ERR_NULL;
  for (int32_t i = 0; i < count; ++i) {
    const fp8_quant_desc_t& d = descs[i];
    if (int st = quantize_checks(d.x, d.dtype, d.n, d.fmt, d.margin, d.y, d.amax, d.bias)) return st;
  }
  if (int st = device_ok()) return st;
  constexpr int kChunk = 256;  // descriptors converted per host batch
  fp8lin::QuantDesc q[kChunk];
  for (int32_t first = 0; first < count; first += kChunk) {
    const int m = count - first < kChunk ? count - first : kChunk;
    for (int i = 0; i < m; ++i) {
      const fp8_quant_desc_t& d = descs[first + i];
      q[i] = fp8lin::QuantDesc{d.x, d.n, d.dtype, d.fmt, d.margin, d.y, d.amax, d.bias};
    }
    if (int st = hip_status(fp8lin::launch_quantize_multi(q, m, (hipStream_t)stream))) return st;
  }
  return FP8_OK;
}

int fp8_scale_cast_amax(const void* x, fp8_dtype_t dtype, int64_t n, const int32_t* bias,
                        fp8_format_t fmt, uint8_t* y, float* x_amax, void* stream) {
  if (n < 0) return FP8_ERR_SIZE;
  if (bad_dtype(dtype)) return FP8_ERR_DTYPE;
  if (bad_format(fmt)) return FP8_ERR_FORMAT;
  if (!x_amax) return FP8_ERR_NULL;
  if (misaligned_word(x_amax)) return FP8_ERR_ALIGN;
  if (n > 0) {
    if (!x || !y || !bias) return FP8_ERR_NULL;
    if (misaligned(x) || misaligned(y) || misaligned_word(bias)) return FP8_ERR_ALIGN;
  }
  if (int s = device_ok()) return s;
  return hip_status(fp8lin::launch_cast(x, dtype, n, bias, fmt, y,
                                        reinterpret_cast<uint32_t*>(x_amax), (hipStream_t)stream));
}

int fp8_quantize_delayed(const void* x, fp8_dtype_t dtype, int64_t n, fp8_format_t fmt,
                         int32_t margin, uint8_t* y, float* amax, int32_t* bias, void* stream) {
  if (int s = quantize_checks(x, dtype, n, fmt, margin, y, amax, bias)) return s;
  if (int s = device_ok()) return s;
  return hip_status(fp8lin::launch_quantize_delayed(x, dtype, n, fmt, margin, y, amax, bias,
                                                    (hipStream_t)stream));
}

}  // extern "C"

namespace {

// The three products; out_amax (optional) receives max |out|.  Every argument
// is checked before any HIP call; on error nothing is written.
// The product's output as rows x cols with contraction `depth`, for each op.
bool out_shape(fp8_gemm_op_t op, int64_t M, int64_t N, int64_t K, int64_t& rows, int64_t& cols,
               int64_t& depth) {
  switch (op) {
    case FP8_GEMM_FWD: rows = M; cols = N; depth = K; return true;
    case FP8_GEMM_DGRAD: rows = M; cols = K; depth = N; return true;
    case FP8_GEMM_WGRAD: rows = N; cols = K; depth = M; return true;
    default: return false;
  }
}

// Where a split product's workspace comes from: none (never split), the
// caller's (fp8_scaled_gemm_ws: ws / ws_bytes checked here) or the library's
// static scratch (fp8_scaled_gemm_noalloc).
enum WsMode { kNoWorkspace, kCallerWorkspace, kStaticScratch };

// The checks of one product and its problem in kernel terms (rows, columns and
// contraction of the output; each operand's layout); empty: no output.
int make_problem(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa, const int32_t* ba,
                 const uint8_t* b, fp8_format_t fb, const int32_t* bb, int64_t M, int64_t N, int64_t K,
                 float* out, fp8lin::GemmProblem& p, bool& empty) {
  if (math != FP8_GEMM_EXACT && math != FP8_GEMM_NATIVE_FP8) return FP8_ERR_OP;
  empty = false;
  switch (op) {
    case FP8_GEMM_FWD:
      // Y[M x N]: X8 and W8 both contraction (K) contiguous.
      if (int s = gemm_checks(a, fa, ba, b, fb, bb, M, N, K, out, M, K, N, K)) return s;
      empty = M == 0 || N == 0;
      p = fp8lin::GemmProblem{a, K, true, fa, ba, b, K, true, fb, bb, out, N,
                              (int)M, (int)N, (int)K, math, nullptr, false};
      break;
    case FP8_GEMM_DGRAD:
      // dX[M x K]: rows of dY8 (contraction N contiguous) times W8 read as
      // [contraction N][K] (the contraction is its slow index).
      if (int s = gemm_checks(a, fa, ba, b, fb, bb, M, K, N, out, M, N, N, K)) return s;
      empty = M == 0 || K == 0;
      p = fp8lin::GemmProblem{a, N, true, fa, ba, b, K, false, fb, bb, out, K,
                              (int)M, (int)K, (int)N, math, nullptr, false};
      break;
    case FP8_GEMM_WGRAD:
      // dW[N x K]: dY8 read as [contraction M][N] times X8 read as [contraction M][K].
      if (int s = gemm_checks(a, fa, ba, b, fb, bb, N, K, M, out, M, N, M, K)) return s;
      empty = N == 0 || K == 0;
      p = fp8lin::GemmProblem{a, N, false, fa, ba, b, K, false, fb, bb, out, K,
                              (int)N, (int)K, (int)M, math, nullptr, false};
      break;
    default:
      return FP8_ERR_OP;
  }
  return FP8_OK;
}

int scaled_gemm(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa, const int32_t* ba,
                const uint8_t* b, fp8_format_t fb, const int32_t* bb, int64_t M, int64_t N,
                int64_t K, float* out, float* out_amax, WsMode ws_mode, void* ws, int64_t ws_bytes,
                hipStream_t st, bool accumulate = false) {
  fp8lin::GemmProblem p{};
  bool empty = false;
  if (int s = make_problem(op, math, a, fa, ba, b, fb, bb, M, N, K, out, p, empty)) return s;
  p.accumulate = accumulate;
  bool split = false;
  // the static scratch bounds its plan; a caller's workspace is sized by
  // fp8_scaled_gemm_workspace_bytes (no bound)
  const int64_t max_bytes = ws_mode == kStaticScratch ? (int64_t)FP8_NOALLOC_SCRATCH_BYTES : INT64_MAX;
  if (ws_mode != kNoWorkspace && !empty) {
    const int64_t need = fp8lin::gemm_split_workspace_bytes(p.m, p.n, p.k, max_bytes);
    if (need > 0) {
      if (ws_mode == kStaticScratch) {
        if (need > (int64_t)FP8_NOALLOC_SCRATCH_BYTES) return FP8_ERR_SIZE;
      } else {
        if (!ws) return FP8_ERR_NULL;
        if (misaligned(ws)) return FP8_ERR_ALIGN;
        if (ws_bytes < need) return FP8_ERR_SIZE;
      }
      split = true;
    }
  }
  if (empty && !out_amax) return FP8_OK;
  if (int s = device_ok()) return s;
  if (split && ws_mode == kStaticScratch) {
    if (int s = scratch_of_current_device(&ws)) return s;
  }
  if (out_amax) {
    p.amax = reinterpret_cast<uint32_t*>(out_amax);
    if (int s = hip_status(fp8lin::launch_clear_u32(p.amax, st))) return s;
  }
  if (empty) return FP8_OK;
  if (split) {
    float* w = static_cast<float*>(ws);
    switch (op) {
      case FP8_GEMM_FWD: return hip_status(fp8lin::launch_gemm_fwd_ws(p, w, max_bytes, st));
      case FP8_GEMM_DGRAD: return hip_status(fp8lin::launch_gemm_dgrad_ws(p, w, max_bytes, st));
      default: return hip_status(fp8lin::launch_gemm_wgrad_ws(p, w, max_bytes, st));
    }
  }
  switch (op) {
    case FP8_GEMM_FWD: return hip_status(fp8lin::launch_gemm_fwd(p, st));
    case FP8_GEMM_DGRAD: return hip_status(fp8lin::launch_gemm_dgrad(p, st));
    default: return hip_status(fp8lin::launch_gemm_wgrad(p, st));
  }
}

// The problems of a group call (checked) and their plan; count products at
// most kGroupMaxProducts.  Returns the workspace bytes (>= 0) or a status.
int64_t group_problems(int math, const fp8_gemm_desc_t* d, int32_t count, fp8lin::GemmProblem* ps,
                       fp8lin::GroupSlot* plan, int* live) {
  if (count < 0 || count > fp8lin::kGroupMaxProducts) return FP8_ERR_SIZE;
  if (count > 0 && !d) return FP8_ERR_NULL;
  *live = 0;
  for (int32_t i = 0; i < count; ++i) {
    bool empty = false;
    fp8lin::GemmProblem p{};
    if (int s = make_problem((fp8_gemm_op_t)d[i].op, math, d[i].a, (fp8_format_t)d[i].fa, d[i].ba, d[i].b,
                             (fp8_format_t)d[i].fb, d[i].bb, d[i].M, d[i].N, d[i].K, d[i].out, p, empty))
      return s;
    if (!empty) ps[(*live)++] = p;
  }
  return fp8lin::gemm_group_plan(ps, *live, plan);
}

}  // namespace

extern "C" {

int64_t fp8_scaled_gemm_group_workspace_bytes(int math, const fp8_gemm_desc_t* descs, int32_t count) {
  fp8lin::GemmProblem ps[fp8lin::kGroupMaxProducts];
  fp8lin::GroupSlot plan[fp8lin::kGroupMaxProducts];
  int live = 0;
  return group_problems(math, descs, count, ps, plan, &live);
}

int fp8_scaled_gemm_group(int math, const fp8_gemm_desc_t* descs, int32_t count, void* ws,
                          int64_t ws_bytes, void* stream) {
  fp8lin::GemmProblem ps[fp8lin::kGroupMaxProducts];
  fp8lin::GroupSlot plan[fp8lin::kGroupMaxProducts];
  int live = 0;
  const int64_t need = group_problems(math, descs, count, ps, plan, &live);
  if (need < 0) return (int)need;
  if (ws_bytes < 0) return FP8_ERR_SIZE;
  if (need > 0) {
    if (!ws) return FP8_ERR_NULL;
    if (misaligned(ws)) return FP8_ERR_ALIGN;
    if (ws_bytes < need) return FP8_ERR_SIZE;
  }
  if (live == 0) return FP8_OK;
  if (int s = device_ok()) return s;
  hipStream_t st = (hipStream_t)stream;
  int idx[3][fp8lin::kGroupMaxProducts];
  int n[3] = {0, 0, 0};
  int step[fp8lin::kGroupMaxProducts];
  int nstep = 0;
  for (int i = 0; i < live; ++i) {
    const fp8lin::GemmProblem& p = ps[i];
    const int layout = p.a_kmajor && p.b_kmajor ? 0 : (p.a_kmajor ? 1 : 2);
    if (plan[i].grouped) {
      if (fp8lin::gemm_step_variant(p) >= 0) step[nstep++] = i;
      else idx[layout][n[layout]++] = i;
      continue;
    }
    hipError_t e = layout == 0 ? fp8lin::launch_gemm_fwd(p, st)
                   : layout == 1 ? fp8lin::launch_gemm_dgrad(p, st) : fp8lin::launch_gemm_wgrad(p, st);
    if (e != hipSuccess) return FP8_ERR_HIP;
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (int s = hip_status(fp8lin::launch_gemm_step_group(ps, plan, step, nstep, w, st))) return s;
  if (int s = hip_status(fp8lin::launch_gemm_fwd_group(ps, plan, idx[0], n[0], w, st))) return s;
  if (int s = hip_status(fp8lin::launch_gemm_dgrad_group(ps, plan, idx[1], n[1], w, st))) return s;
  return hip_status(fp8lin::launch_gemm_wgrad_group(ps, plan, idx[2], n[2], w, st));
}

int fp8_scaled_gemm(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                    const int32_t* ba, const uint8_t* b, fp8_format_t fb, const int32_t* bb,
                    int64_t M, int64_t N, int64_t K, float* out, void* stream) {
  return scaled_gemm(op, math, a, fa, ba, b, fb, bb, M, N, K, out, nullptr, kNoWorkspace, nullptr,
                     0, (hipStream_t)stream);
}

int64_t fp8_scaled_gemm_workspace_bytes(fp8_gemm_op_t op, int64_t M, int64_t N, int64_t K) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return FP8_ERR_SIZE;
  int64_t rows, cols, depth;
  if (!out_shape(op, M, N, K, rows, cols, depth)) return FP8_ERR_OP;
  return fp8lin::gemm_split_workspace_bytes(rows, cols, depth, INT64_MAX);
}

int fp8_scaled_gemm_ws(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                       const int32_t* ba, const uint8_t* b, fp8_format_t fb, const int32_t* bb,
                       int64_t M, int64_t N, int64_t K, float* out, void* ws, int64_t ws_bytes,
                       void* stream) {
  if (ws_bytes < 0) return FP8_ERR_SIZE;
  return scaled_gemm(op, math, a, fa, ba, b, fb, bb, M, N, K, out, nullptr, kCallerWorkspace, ws,
                     ws_bytes, (hipStream_t)stream);
}

int fp8_scaled_gemm_noalloc(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                            const int32_t* ba, const uint8_t* b, fp8_format_t fb,
                            const int32_t* bb, int64_t M, int64_t N, int64_t K, float* out,
                            void* stream) {
  return scaled_gemm(op, math, a, fa, ba, b, fb, bb, M, N, K, out, nullptr, kStaticScratch,
                     nullptr, 0, (hipStream_t)stream);
}

int fp8_scaled_gemm_amax(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                         const int32_t* ba, const uint8_t* b, fp8_format_t fb, const int32_t* bb,
                         int64_t M, int64_t N, int64_t K, float* out, float* out_amax,
                         void* stream) {
  if (!out_amax) return FP8_ERR_NULL;
  if (misaligned_word(out_amax)) return FP8_ERR_ALIGN;
  return scaled_gemm(op, math, a, fa, ba, b, fb, bb, M, N, K, out, out_amax, kNoWorkspace, nullptr,
                     0, (hipStream_t)stream);
}

int fp8_scaled_gemm_accumulate(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                               const int32_t* ba, const uint8_t* b, fp8_format_t fb,
                               const int32_t* bb, int64_t M, int64_t N, int64_t K, float* out,
                               void* stream) {
  return scaled_gemm(op, math, a, fa, ba, b, fb, bb, M, N, K, out, nullptr, kNoWorkspace, nullptr,
                     0, (hipStream_t)stream, true);
}

int fp8_scaled_gemm_fwd(const uint8_t* x8, fp8_format_t fx, const int32_t* bx,
                        const uint8_t* w8, fp8_format_t fw, const int32_t* bw, int64_t M,
                        int64_t N, int64_t K, float* y, void* stream) {
  return fp8_scaled_gemm(FP8_GEMM_FWD, FP8_GEMM_EXACT, x8, fx, bx, w8, fw, bw, M, N, K, y, stream);
}

int fp8_scaled_gemm_dgrad(const uint8_t* dy8, fp8_format_t fdy, const int32_t* bdy,
                          const uint8_t* w8, fp8_format_t fw, const int32_t* bw, int64_t M,
                          int64_t N, int64_t K, float* dx, void* stream) {
  return fp8_scaled_gemm(FP8_GEMM_DGRAD, FP8_GEMM_EXACT, dy8, fdy, bdy, w8, fw, bw, M, N, K, dx,
                         stream);
}

int fp8_scaled_gemm_wgrad(const uint8_t* dy8, fp8_format_t fdy, const int32_t* bdy,
                          const uint8_t* x8, fp8_format_t fx, const int32_t* bx, int64_t M,
                          int64_t N, int64_t K, float* dw, void* stream) {
  return fp8_scaled_gemm(FP8_GEMM_WGRAD, FP8_GEMM_EXACT, dy8, fdy, bdy, x8, fx, bx, M, N, K, dw,
                         stream);
}

}  // extern "C"

namespace {

int swiglu_checks(const void* h, const void* da, bool need_da, int64_t rows, int64_t f,
                  const void* out, const float* out_amax) {
  if (rows < 0 || f < 0 || rows > (int64_t)0x7FFFFFFF || f > (int64_t)0x3FFFFFFF)
    return FP8_ERR_SIZE;
  if (fp8lin::swiglu_blocks(rows, f) > (int64_t)0x7FFFFFFF) return FP8_ERR_SIZE;
  if (out_amax && misaligned_word(out_amax)) return FP8_ERR_ALIGN;
  if (rows == 0 || f == 0) return FP8_OK;
  if (!h || !out || (need_da && !da)) return FP8_ERR_NULL;
  if (misaligned(h) || misaligned(out) || (need_da && misaligned(da))) return FP8_ERR_ALIGN;
  return FP8_OK;
}

}  // namespace

extern "C" {

int fp8_swiglu_fwd(const float* h, int64_t rows, int64_t f, uint16_t* a, float* out_amax,
                   void* stream) {
  if (int s = swiglu_checks(h, nullptr, false, rows, f, a, out_amax)) return s;
  if ((rows == 0 || f == 0) && !out_amax) return FP8_OK;
  if (int s = device_ok()) return s;
  return hip_status(fp8lin::launch_swiglu_fwd(h, rows, f, a, reinterpret_cast<uint32_t*>(out_amax),
                                              (hipStream_t)stream));
}

int fp8_swiglu_bwd(const float* h, const float* da, int64_t rows, int64_t f, uint16_t* dh,
                   float* out_amax, void* stream) {
  if (int s = swiglu_checks(h, da, true, rows, f, dh, out_amax)) return s;
  if ((rows == 0 || f == 0) && !out_amax) return FP8_OK;
  if (int s = device_ok()) return s;
  return hip_status(fp8lin::launch_swiglu_bwd(h, da, rows, f, dh,
                                              reinterpret_cast<uint32_t*>(out_amax),
                                              (hipStream_t)stream));
}

}  // extern "C"
