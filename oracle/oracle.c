/*
 * CPU oracle for the FP8-AMAX scaled linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, scalar definition
 * that the HIP library is checked against.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg load it.  It shares no code, header, table
 * or constant generator with the HIP path, and it never calls that path.
 *
 * What it follows.  "Training and inference of large language models using
 * 8-bit floating point" (Perez, Zhang et al., 2023), review page, section
 * "Proposed method" (bullets 1-4):
 *   - the scale of each weight, activation and gradient tensor comes from the
 *     tensor's maximum absolute value (bullet 1);
 *   - compute_bias takes log2 of (format maximum / tensor amplitude) and a
 *     configurable margin (bullet 2);
 *   - the input is scaled before the cast to FP8 and the matmul result is
 *     unscaled afterwards (bullet 3);
 *   - FP8_E4 holds weights and activations, FP8_E5 holds gradients (bullet 4).
 *
 * Readings where the page is silent (each is listed in the design notes):
 *   - FP8_E4 / FP8_E5 are the OCP 8-bit formats E4M3 (max 448, no infinity,
 *     NaN = S.1111.111) and E5M2 (max 57344, IEEE-style inf and NaN);
 *   - E3M4, the third format of the post-training quantisation study ("Efficient
 *     post-training quantization with FP8 formats", summary page), is named
 *     there without its encoding; it is read here as built like OCP E4M3:
 *     exponent bias 3, 4 mantissa bits, subnormals, no infinity, NaN only at
 *     S.111.1111, so max 30 = S.111.1110 and the smallest subnormal 2^-6;
 *   - bias = floor(log2(fmt_max / amax)) - margin, an integer, so the scale
 *     2^bias is a power of two and amax * 2^bias <= fmt_max when margin >= 0;
 *   - amax that is 0, inf or NaN gives bias 0 and the margin is not applied;
 *   - the cast rounds to nearest, ties to the even code, saturates finite and
 *     infinite overflow to the largest finite code, keeps FP8 subnormals,
 *     keeps the sign of zero, and maps NaN to code 0x7F with the input's sign;
 *   - amax of a tensor holding NaN is the NaN whose magnitude bits are largest;
 *     amax of an empty tensor is 0;
 *   - the matmul result is sum_k a_k * b_k over the decoded FP8 values times
 *     2^-(bias_a + bias_b); here it is formed in fp64, in ascending k;
 *   - the activation between the products of a chained MLP is Llama 2's gated
 *     SwiGLU (the pages train Llama 2 models, "Main findings", but do not
 *     spell the activation out): a = silu(g) * u with silu(g) = g * sigmoid(g),
 *     where g and u are the two halves of the up-projection's output.
 *
 * Every finite input is decoded into an exact triple (sign, integer
 * significand S, power-of-two exponent q) with value (-1)^sign * S * 2^q, so
 * no step below rounds except the one rounding the cast defines.
 *
 * Pins: tests/test_oracle_*.py check every function here against brute force,
 * a library routine or a closed form; none is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_F32 1
#define ORACLE_E4M3 0
#define ORACLE_E5M2 1
#define ORACLE_E3M4 2

/* Threads the OpenMP loops below may use (1 without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

enum { CLS_ZERO = 0, CLS_FINITE = 1, CLS_INF = 2, CLS_NAN = 3 };

typedef struct {
  int cls;       /* CLS_* */
  int sign;      /* 1 if negative */
  uint64_t sig;  /* integer significand S (>0 when CLS_FINITE) */
  int exp;       /* value = S * 2^exp */
  uint32_t mag;  /* magnitude bits, in fp32 layout (NaN payload order) */
} exact_t;

/* bf16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
static exact_t decode_bf16(uint16_t h) {
  exact_t r;
  unsigned e = (h >> 7) & 0xFF, m = h & 0x7F;
  r.sign = h >> 15;
  r.mag = (uint32_t)(h & 0x7FFF) << 16;
  r.sig = 0;
  r.exp = 0;
  if (e == 0xFF) {
    r.cls = m ? CLS_NAN : CLS_INF;
  } else if (e == 0) {
    r.cls = m ? CLS_FINITE : CLS_ZERO;
    r.sig = m;          /* subnormal: m * 2^(1-127-7) */
    r.exp = -133;
  } else {
    r.cls = CLS_FINITE;
    r.sig = 128u + m;   /* normal: (1.m) * 2^(e-127) = (128+m) * 2^(e-134) */
    r.exp = (int)e - 134;
  }
  return r;
}

/* fp32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits. */
static exact_t decode_f32(uint32_t u) {
  exact_t r;
  unsigned e = (u >> 23) & 0xFF, m = u & 0x7FFFFF;
  r.sign = u >> 31;
  r.mag = u & 0x7FFFFFFFu;
  r.sig = 0;
  r.exp = 0;
  if (e == 0xFF) {
    r.cls = m ? CLS_NAN : CLS_INF;
  } else if (e == 0) {
    r.cls = m ? CLS_FINITE : CLS_ZERO;
    r.sig = m;
    r.exp = -149;
  } else {
    r.cls = CLS_FINITE;
    r.sig = (1u << 23) + m;
    r.exp = (int)e - 150;
  }
  return r;
}

static exact_t decode_input(const void* x, int dtype, int64_t i) {
  if (dtype == ORACLE_BF16) return decode_bf16(((const uint16_t*)x)[i]);
  return decode_f32(((const uint32_t*)x)[i]);
}

/* Exact magnitude as a double (bf16 and fp32 values are all exact in fp64). */
static double magnitude(exact_t v) { return ldexp((double)v.sig, v.exp); }

/* ------------------------------------------------------------------------
 * Step 1: per-tensor maximum absolute value ("Proposed method", bullet 1).
 * Returns the fp32 bit pattern of max_i |x_i|.  A bf16 value widens to fp32
 * exactly.  NaN anywhere gives the NaN of largest magnitude bits; otherwise an
 * infinity gives +inf; an empty tensor gives +0.
 * ---------------------------------------------------------------------- */
uint32_t oracle_amax(const void* x, int dtype, int64_t n) {
  double best = 0.0;
  int any_inf = 0, any_nan = 0;
  uint32_t nan_mag = 0;
  for (int64_t i = 0; i < n; ++i) {
    exact_t v = decode_input(x, dtype, i);
    if (v.cls == CLS_NAN) {
      any_nan = 1;
      if (v.mag > nan_mag) nan_mag = v.mag;
    } else if (v.cls == CLS_INF) {
      any_inf = 1;
    } else if (v.cls == CLS_FINITE) {
      double a = magnitude(v);
      if (a > best) best = a;
    }
  }
  if (any_nan) return nan_mag;
  if (any_inf) return 0x7F800000u;
  float f = (float)best; /* exact: best is one of the inputs' magnitudes */
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return bits;
}

/* Format parameters of the OCP 8-bit floats. */
typedef struct {
  int mbits;       /* stored mantissa bits */
  int emin;        /* exponent of the smallest normal binade */
  int emax;        /* exponent of the largest finite binade */
  double fmt_max;  /* largest finite magnitude */
  unsigned maxcode;/* code of +fmt_max */
} fmt_t;

static fmt_t format_params(int fmt) {
  fmt_t f;
  if (fmt == ORACLE_E4M3) {
    f.mbits = 3; f.emin = -6; f.emax = 8; f.fmt_max = 448.0; f.maxcode = 0x7E;
  } else if (fmt == ORACLE_E5M2) {
    f.mbits = 2; f.emin = -14; f.emax = 15; f.fmt_max = 57344.0; f.maxcode = 0x7B;
  } else {
    f.mbits = 4; f.emin = -2; f.emax = 4; f.fmt_max = 30.0; f.maxcode = 0x7E;
  }
  return f;
}

/* ------------------------------------------------------------------------
 * Step 2: compute_bias ("Proposed method", bullet 2):
 *   bias = floor(log2(fmt_max / amax)) - margin.
 * Evaluated exactly.  With amax = f * 2^e and fmt_max = fm * 2^em (frexp, so
 * f and fm lie in [0.5, 1)), fmt_max/amax = (fm/f) * 2^(em-e) and fm/f lies in
 * (0.5, 2): its floor(log2) is -1 when f > fm and 0 otherwise.
 * amax of 0, inf or NaN: bias 0, margin not applied.
 * ---------------------------------------------------------------------- */
int32_t oracle_compute_bias(uint32_t amax_bits, int fmt, int32_t margin) {
  float a;
  memcpy(&a, &amax_bits, sizeof a);
  if (!(a > 0.0f) || isinf(a)) return 0; /* zero, negative zero, NaN or inf */
  fmt_t F = format_params(fmt);
  int e, em;
  double f = frexp((double)a, &e);
  double fm = frexp(F.fmt_max, &em);
  int floor_log2 = (em - e) - (f > fm ? 1 : 0);
  return (int32_t)(floor_log2 - margin);
}

/* Exact FP8 value of a code. */
double oracle_decode_fp8(uint8_t c, int fmt) {
  int s = c >> 7;
  double v;
  if (fmt == ORACLE_E4M3) {
    int E = (c >> 3) & 15, M = c & 7;
    if (E == 15 && M == 7) return NAN;
    v = (E == 0) ? ldexp((double)M, -9) : ldexp((double)(8 + M), E - 10);
  } else if (fmt == ORACLE_E3M4) {
    int E = (c >> 4) & 7, M = c & 15;
    if (E == 7 && M == 15) return NAN;
    v = (E == 0) ? ldexp((double)M, -6) : ldexp((double)(16 + M), E - 7);
  } else {
    int E = (c >> 2) & 31, M = c & 3;
    if (E == 31) return M ? NAN : (s ? -INFINITY : INFINITY);
    v = (E == 0) ? ldexp((double)M, -16) : ldexp((double)(4 + M), E - 17);
  }
  return s ? -v : v;
}

static int bit_length(uint64_t s) {
  int b = 0;
  while (s) { ++b; s >>= 1; }
  return b;
}

/* Round the exact value S * 2^q (S > 0) to the format's grid, ties to the
 * even code, saturating at fmt_max.  Returns the magnitude code. */
static unsigned encode_magnitude(uint64_t S, int q, fmt_t F) {
  int t = bit_length(S) - 1 + q;        /* floor(log2(value)) */
  if (t > F.emax) return F.maxcode;     /* at least 2^(emax+1) > fmt_max */
  int Qe = (t < F.emin ? F.emin : t) - F.mbits; /* exponent of one ulp here */
  int sh = Qe - q;                      /* value / 2^Qe = S * 2^(-sh) */
  uint64_t n;
  if (sh <= 0) {
    n = S << (-sh);                     /* exact; n < 2^(mbits+1) */
  } else if (sh >= 63) {
    n = 0;                              /* S < 2^62 = half an ulp */
  } else {
    n = S >> sh;
    uint64_t rem = S & ((1ull << sh) - 1);
    uint64_t half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (n & 1))) n += 1;
  }
  unsigned c;
  if (t < F.emin) {
    c = (unsigned)n;                    /* subnormal: n ulps of 2^(emin-mbits) */
  } else {                              /* normal: n in [2^mbits, 2^(mbits+1)] */
    c = ((unsigned)(t - F.emin + 1) << F.mbits) + (unsigned)(n - (1ull << F.mbits));
  }
  if (c > F.maxcode) c = F.maxcode;     /* saturate */
  return c;
}

static uint8_t encode_scaled(exact_t v, int32_t bias, fmt_t F) {
  unsigned s = (unsigned)v.sign << 7;
  switch (v.cls) {
    case CLS_NAN: return (uint8_t)(0x7F | s);
    case CLS_INF: return (uint8_t)(F.maxcode | s);
    case CLS_ZERO: return (uint8_t)s;
    default: return (uint8_t)(encode_magnitude(v.sig, v.exp + bias, F) | s);
  }
}

/* ------------------------------------------------------------------------
 * Step 3: scale by 2^bias, then cast ("Proposed method", bullets 3-4).
 * y[i] = code nearest to x[i] * 2^bias (exact product), see encode_magnitude.
 * ---------------------------------------------------------------------- */
void oracle_scale_cast(const void* x, int dtype, int64_t n, int32_t bias, int fmt,
                       uint8_t* y) {
  fmt_t F = format_params(fmt);
  for (int64_t i = 0; i < n; ++i) y[i] = encode_scaled(decode_input(x, dtype, i), bias, F);
}

/* ------------------------------------------------------------------------
 * Step 4: FP8 x FP8 matmul, then unscale ("Proposed method", bullet 3).
 * out = 2^-(ba+bb) * sum over the contraction index of deq(a) * deq(b),
 * summed in fp64 in ascending contraction index.  bound = 2^-(ba+bb) *
 * sum |deq(a)| * |deq(b)| is the scale the tolerance is taken against.
 *
 *   fwd:   Y[i][j]  = sum_k X8[i][k]  * W8[j][k]   X8: MxK, W8: NxK, Y: MxN
 *   dgrad: dX[i][k] = sum_j dY8[i][j] * W8[j][k]   dY8: MxN, W8: NxK, dX: MxK
 *   wgrad: dW[j][k] = sum_i dY8[i][j] * X8[i][k]   dY8: MxN, X8: MxK, dW: NxK
 * All matrices are row-major.  Either output pointer may be NULL.
 * ---------------------------------------------------------------------- */
static void decode_table(int fmt, double* t) {
  for (int c = 0; c < 256; ++c) t[c] = oracle_decode_fp8((uint8_t)c, fmt);
}

void oracle_gemm_fwd(const uint8_t* x8, int fx, int32_t bx, const uint8_t* w8, int fw,
                     int32_t bw, int64_t M, int64_t N, int64_t K, double* y, double* bound) {
  double tx[256], tw[256];
  decode_table(fx, tx);
  decode_table(fw, tw);
  int unscale = -(bx + bw);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double a = tx[x8[i * K + k]], b = tw[w8[j * K + k]];
        acc += a * b;
        mag += fabs(a) * fabs(b);
      }
      if (y) y[i * N + j] = ldexp(acc, unscale);
      if (bound) bound[i * N + j] = ldexp(mag, unscale);
    }
  }
}

void oracle_gemm_dgrad(const uint8_t* dy8, int fdy, int32_t bdy, const uint8_t* w8, int fw,
                       int32_t bw, int64_t M, int64_t N, int64_t K, double* dx, double* bound) {
  double ta[256], tb[256];
  decode_table(fdy, ta);
  decode_table(fw, tb);
  int unscale = -(bdy + bw);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0, mag = 0.0;
      for (int64_t j = 0; j < N; ++j) {
        double a = ta[dy8[i * N + j]], b = tb[w8[j * K + k]];
        acc += a * b;
        mag += fabs(a) * fabs(b);
      }
      if (dx) dx[i * K + k] = ldexp(acc, unscale);
      if (bound) bound[i * K + k] = ldexp(mag, unscale);
    }
  }
}

void oracle_gemm_wgrad(const uint8_t* dy8, int fdy, int32_t bdy, const uint8_t* x8, int fx,
                       int32_t bx, int64_t M, int64_t N, int64_t K, double* dw, double* bound) {
  double ta[256], tb[256];
  decode_table(fdy, ta);
  decode_table(fx, tb);
  int unscale = -(bdy + bx);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < N; ++j) {
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0, mag = 0.0;
      for (int64_t i = 0; i < M; ++i) {
        double a = ta[dy8[i * N + j]], b = tb[x8[i * K + k]];
        acc += a * b;
        mag += fabs(a) * fabs(b);
      }
      if (dw) dw[j * K + k] = ldexp(acc, unscale);
      if (bound) bound[j * K + k] = ldexp(mag, unscale);
    }
  }
}

/* The same three products evaluated only at the listed output positions
 * (row[t], col[t]) -- used where the full output is too large for the CPU. */
void oracle_gemm_fwd_at(const uint8_t* x8, int fx, int32_t bx, const uint8_t* w8, int fw,
                        int32_t bw, int64_t M, int64_t N, int64_t K, const int64_t* row,
                        const int64_t* col, int64_t cnt, double* out, double* bound) {
  double tx[256], tw[256];
  decode_table(fx, tx);
  decode_table(fw, tw);
  int unscale = -(bx + bw);
  (void)M; (void)N;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < cnt; ++t) {
    int64_t i = row[t], j = col[t];
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double a = tx[x8[i * K + k]], b = tw[w8[j * K + k]];
      acc += a * b;
      mag += fabs(a) * fabs(b);
    }
    out[t] = ldexp(acc, unscale);
    if (bound) bound[t] = ldexp(mag, unscale);
  }
}

void oracle_gemm_dgrad_at(const uint8_t* dy8, int fdy, int32_t bdy, const uint8_t* w8, int fw,
                          int32_t bw, int64_t M, int64_t N, int64_t K, const int64_t* row,
                          const int64_t* col, int64_t cnt, double* out, double* bound) {
  double ta[256], tb[256];
  decode_table(fdy, ta);
  decode_table(fw, tb);
  int unscale = -(bdy + bw);
  (void)M;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < cnt; ++t) {
    int64_t i = row[t], k = col[t];
    double acc = 0.0, mag = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      double a = ta[dy8[i * N + j]], b = tb[w8[j * K + k]];
      acc += a * b;
      mag += fabs(a) * fabs(b);
    }
    out[t] = ldexp(acc, unscale);
    if (bound) bound[t] = ldexp(mag, unscale);
  }
}

void oracle_gemm_wgrad_at(const uint8_t* dy8, int fdy, int32_t bdy, const uint8_t* x8, int fx,
                          int32_t bx, int64_t M, int64_t N, int64_t K, const int64_t* row,
                          const int64_t* col, int64_t cnt, double* out, double* bound) {
  double ta[256], tb[256];
  decode_table(fdy, ta);
  decode_table(fx, tb);
  int unscale = -(bdy + bx);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < cnt; ++t) {
    int64_t j = row[t], k = col[t];
    double acc = 0.0, mag = 0.0;
    for (int64_t i = 0; i < M; ++i) {
      double a = ta[dy8[i * N + j]], b = tb[x8[i * K + k]];
      acc += a * b;
      mag += fabs(a) * fabs(b);
    }
    out[t] = ldexp(acc, unscale);
    if (bound) bound[t] = ldexp(mag, unscale);
  }
}

/* ------------------------------------------------------------------------
 * Step 5: the gated activation between the two products of a chained MLP
 * (SwiGLU, the reading in the header), in fp64.
 *   h:  rows x 2f fp32, row t = [g_t0 .. g_t(f-1) | u_t0 .. u_t(f-1)]
 *   forward   a[t][j]        = silu(g) * u
 *   backward  dh[t][j]       = da * u * silu'(g)   (d a / d g)
 *             dh[t][f + j]   = da * silu(g)        (d a / d u)
 * with sigmoid(g) = 1 / (1 + e^-g), silu(g) = g * sigmoid(g) and
 * silu'(g) = sigmoid(g) * (1 + g * (1 - sigmoid(g))).  sigmoid and
 * 1 - sigmoid are taken from e^-|g| (e / (1 + e) and 1 / (1 + e)), the same
 * values without forming 1 - sigmoid by subtraction.
 * ---------------------------------------------------------------------- */
static void sigmoid_pair(double g, double* s, double* sc) {
  if (g < 0.0) {
    double e = exp(g);
    *s = e / (1.0 + e);
    *sc = 1.0 / (1.0 + e);
  } else {
    double e = exp(-g);
    *s = 1.0 / (1.0 + e);
    *sc = e / (1.0 + e);
  }
}

void oracle_swiglu_fwd(const float* h, int64_t rows, int64_t f, double* a) {
  for (int64_t t = 0; t < rows; ++t)
    for (int64_t j = 0; j < f; ++j) {
      double g = h[t * 2 * f + j], u = h[t * 2 * f + f + j], s, sc;
      sigmoid_pair(g, &s, &sc);
      a[t * f + j] = g * s * u;
    }
}

void oracle_swiglu_bwd(const float* h, const float* da, int64_t rows, int64_t f, double* dh) {
  for (int64_t t = 0; t < rows; ++t)
    for (int64_t j = 0; j < f; ++j) {
      double g = h[t * 2 * f + j], u = h[t * 2 * f + f + j], d = da[t * f + j], s, sc;
      sigmoid_pair(g, &s, &sc);
      dh[t * 2 * f + j] = d * u * (s * (1.0 + g * sc));
      dh[t * 2 * f + f + j] = d * (g * s);
    }
}
