/*
 * fp8lin -- FP8-AMAX scaled linear layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the native library (libfp8lin.so).  Plain pointers and sizes only.
 *
 * The method: "Training and inference of large language models using 8-bit
 * floating point" (Perez, Zhang et al., 2023), review page, section "Proposed
 * method".  Each weight, activation and gradient tensor gets a per-tensor scale
 * from its maximum absolute value (bullet 1); compute_bias turns that value
 * into a power-of-two exponent from log2(format max / amplitude) with a
 * configurable margin (bullet 2); the tensor is scaled before the FP8 cast and
 * the matmul result is unscaled afterwards (bullet 3); weights and activations
 * use E4 (E4M3), gradients E5 (E5M2) (bullet 4); the same products serve
 * training (forward, data gradient, weight gradient) and post-training
 * quantised inference (bullet 5).
 *
 * Conventions for every entry point:
 *  - Device pointers are device memory of the current HIP device (for example
 *    torch.empty(..., device="cuda").data_ptr()).  The caller allocates every
 *    buffer; the library never allocates, frees or keeps a pointer (its one
 *    piece of device memory is the static scratch of fp8_scaled_gemm_noalloc).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it and the call returns without waiting; nothing is copied to the host.
 *  - Matrices are row-major and dense (leading dimension = column count).
 *  - Arguments are checked on the host before any HIP call; on error the call
 *    returns a negative status synchronously and leaves every output untouched.
 *    A launch failure returns FP8_ERR_HIP; a fault during execution surfaces at
 *    the caller's next synchronisation.
 *  - Calls are thread-safe.  Calls that write the same output must not overlap
 *    (nor, on one GPU, two fp8_scaled_gemm_noalloc calls).
 *  - Tuning only (read at each call, never needed for correct results):
 *    FP8LIN_GEMM_TILE=128|256 forces the products' tile, FP8LIN_EXACT_MFMA=
 *    f16|bf16 the 16-bit MFMA of the exact arithmetic, FP8LIN_AMAX_HINT /
 *    FP8LIN_CAST_HINT=cached ordinary instead of streaming loads,
 *    FP8LIN_QUANT_SMALL=n the largest tensor (elements) fp8_quantize does in
 *    one workgroup, and FP8LIN_SPLIT_SLOTS=n the workgroup slots the split of
 *    fp8_scaled_gemm_ws plans for (256; it also changes the workspace size).
 */
#ifndef FP8LIN_H
#define FP8LIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FP8 encodings.  E4M3 and E5M2 are the OCP 8-bit formats, the review page's
 * FP8_E4 and FP8_E5.  E3M4 is the third format of the post-training
 * quantisation study ("Efficient post-training quantization with FP8
 * formats", summary page), which names it without an encoding; it is built
 * here like OCP E4M3.  E3M4 is accepted by fp8_compute_bias and
 * fp8_scale_cast only: gfx950's MFMA has no E3M4 operand, so the products
 * reject it with FP8_ERR_FORMAT. */
typedef enum {
  FP8_E4M3 = 0, /* 1-4-3, exponent bias 7, max 448, no infinity, NaN = S.1111.111 */
  FP8_E5M2 = 1, /* 1-5-2, exponent bias 15, max 57344, inf = S.11111.00 (never produced) */
  FP8_E3M4 = 2  /* 1-3-4, exponent bias 3, max 30, no infinity, NaN = S.111.1111 */
} fp8_format_t;

/* Element type of a high-precision input tensor. */
typedef enum {
  FP8_IN_BF16 = 0, /* 2-byte bfloat16 */
  FP8_IN_FP32 = 1  /* 4-byte IEEE binary32 */
} fp8_dtype_t;

/* Status codes. */
#define FP8_OK 0
#define FP8_ERR_NULL (-1)   /* a required pointer is NULL */
#define FP8_ERR_SIZE (-2)   /* a size is negative or too large */
#define FP8_ERR_FORMAT (-3) /* format is not an fp8_format_t (or E3M4 given to a product) */
#define FP8_ERR_DTYPE (-4)  /* dtype is not an fp8_dtype_t */
#define FP8_ERR_ALIGN (-5)  /* a pointer is misaligned: tensors need 16 bytes, amax outputs 4 */
#define FP8_ERR_MARGIN (-6) /* |margin| > FP8_MAX_MARGIN */
#define FP8_ERR_DEVICE (-7) /* no HIP device, or the current device is not gfx950 */
#define FP8_ERR_HIP (-8)    /* a HIP launch failed */
#define FP8_ERR_OP (-9)     /* unknown product or math selector */

#define FP8_MAX_MARGIN 64

/* Human-readable name of a status code (static string, never NULL). */
const char* fp8_status_string(int status);

/*
 * Per-tensor maximum absolute value ("Proposed method", bullet 1).
 *   x     device, n elements of `dtype`, 16-byte aligned.
 *   amax  device, one float, 4-byte aligned: written with max_i |x_i|.  The result is exact
 *         (a bf16 value widens to float without rounding).  Any NaN element
 *         makes it the NaN with the largest magnitude bits; otherwise any
 *         infinity makes it +inf; n == 0 gives +0.
 * Two launches on `stream`: one clearing *amax, one reduction.
 */
int fp8_amax(const void* x, fp8_dtype_t dtype, int64_t n, float* amax, void* stream);

/*
 * Scaling bias ("Proposed method", bullet 2): the largest integer b with
 * amax * 2^b <= fmt_max, minus `margin`, i.e. floor(log2(fmt_max/amax)) - margin,
 * evaluated exactly from the exponent and mantissa fields.  fmt_max is 448
 * (E4M3), 57344 (E5M2) or 30 (E3M4).  An amax of 0, inf or NaN gives b = 0 and the margin
 * is not applied.
 *   amax  device, one float, 4-byte aligned (normally the output of fp8_amax).
 *   bias  device, one int32, 4-byte aligned, written.
 *   |margin| <= FP8_MAX_MARGIN; a positive margin leaves headroom below
 *   fmt_max, a negative one makes the largest values saturate.
 */
int fp8_compute_bias(const float* amax, fp8_format_t fmt, int32_t margin, int32_t* bias,
                     void* stream);

/*
 * Scale then cast ("Proposed method", bullets 3-4): y[i] = FP8 code nearest to
 * x[i] * 2^bias.  The product is exact; rounding is to nearest with ties to the
 * even code; magnitudes beyond fmt_max and infinities saturate to the largest
 * finite code; FP8 subnormals are produced; zero and underflow keep the sign
 * (-0 is 0x80); NaN becomes 0x7F | sign.
 *   x     device, n elements of `dtype`, 16-byte aligned.
 *   bias  device, one int32, 4-byte aligned (normally the output of
 *         fp8_compute_bias).
 *   y     device, n bytes, 16-byte aligned, written.
 */
int fp8_scale_cast(const void* x, fp8_dtype_t dtype, int64_t n, const int32_t* bias,
                   fp8_format_t fmt, uint8_t* y, void* stream);

/*
 * The whole per-tensor quantisation ("Proposed method", bullets 1-4):
 * fp8_amax, fp8_compute_bias and fp8_scale_cast in one call, with the same
 * results bit for bit, in fewer launches.  Inputs of up to 256 KiB (131072
 * bf16 or 65536 fp32 elements) take one launch of one workgroup; larger ones
 * three (a one-lane clear of amax, the amax reduction, and the cast, every
 * block of which derives the bias from the amax itself).
 *   x      device, n elements of `dtype`, 16-byte aligned.
 *   y      device, n bytes, 16-byte aligned, written with the codes.
 *   amax   device, one float, 4-byte aligned, written as by fp8_amax.
 *   bias   device, one int32, 4-byte aligned, written as by fp8_compute_bias.
 *   |margin| <= FP8_MAX_MARGIN (FP8_ERR_MARGIN otherwise).
 * n == 0 writes amax = 0 and bias = 0.  Errors as for the three calls.
 */
int fp8_quantize(const void* x, fp8_dtype_t dtype, int64_t n, fp8_format_t fmt, int32_t margin,
                 uint8_t* y, float* amax, int32_t* bias, void* stream);

/*
 * fp8_scale_cast that also returns max |x| of its own input, folded in the
 * same pass ("Proposed method", bullet 1, fused with the cast): with delayed
 * scaling -- this call's bias computed from the amax that the previous call
 * on the previous step's tensor returned -- every quantisation reads its
 * input once (3 bytes per bf16 element instead of amax + cast's 5).
 *   x_amax  device, one float, 4-byte aligned, written: bit-identical to
 *           fp8_amax over x (0 for n == 0).
 * The codes are those of fp8_scale_cast.  Two launches and no atomics: the
 * cast of all but a last stretch of x, each workgroup leaving its largest
 * magnitude as a word in the code bytes of that stretch, then one workgroup
 * that reduces those words and casts the stretch over them (one launch of one
 * workgroup alone for inputs up to 256 KiB).  Returns FP8_ERR_NULL /
 * FP8_ERR_ALIGN for a null or misaligned x_amax, otherwise as fp8_scale_cast.
 */
int fp8_scale_cast_amax(const void* x, fp8_dtype_t dtype, int64_t n, const int32_t* bias,
                        fp8_format_t fmt, uint8_t* y, float* x_amax, void* stream);

/*
 * Delayed scaling of one tensor in one call ("Proposed method", bullets 1-2,
 * with the scale taken from the previous step's amax): bias =
 * fp8_compute_bias(amax, fmt, margin) from the amax the previous step left in
 * *amax, the cast at that bias (codes as fp8_scale_cast), and then max |x| of
 * this input into *amax for the next step -- fp8_compute_bias followed by
 * fp8_scale_cast_amax, bit for bit, without the bias's own launch.
 *   amax  device, one float, 4-byte aligned: read (the previous step's amax;
 *         0 gives bias 0), then overwritten with max |x| (as fp8_amax).
 *   bias  device, one int32, 4-byte aligned, written with the bias used.
 *   x, y, margin as for fp8_quantize.
 * Two launches, as fp8_scale_cast_amax (one for inputs up to 256 KiB); every
 * workgroup derives the bias from *amax, which only the last one overwrites,
 * at its end.  n == 0 writes the bias and amax = 0.  Errors as fp8_quantize.
 */
int fp8_quantize_delayed(const void* x, fp8_dtype_t dtype, int64_t n, fp8_format_t fmt,
                         int32_t margin, uint8_t* y, float* amax, int32_t* bias, void* stream);

/*
 * fp8_quantize_multi: fp8_quantize of several tensors in one call -- the
 * per-tensor amax, bias and cast of "Proposed method", bullets 1-4, for each
 * tensor on its own -- so that a step that quantises many tensors (a layer's
 * activations, weights and gradients) pays a few kernel dispatches instead of
 * up to three per tensor: tensors of at most 256 KiB are quantised by one
 * workgroup each, 32 tensors per launch; the others take three launches per
 * 32 tensors (one clears every amax, one reduces every tensor's amax, one
 * casts every tensor deriving its bias from its amax).
 *   descs  host array of count descriptors (read during the call only):
 *          x, n, dtype, fmt, margin, y, amax, bias exactly as fp8_quantize's
 *          arguments for that tensor.  The outputs of different tensors must
 *          not overlap one another or any input.
 *   count  >= 0 (0: nothing is launched).
 * Each tensor's amax, bias and codes are bit-identical to fp8_quantize on it
 * alone.  Every descriptor is checked before anything is launched; the first
 * bad one's status is returned (as fp8_quantize would return it), and nothing
 * runs.  FP8_ERR_NULL for descs == NULL with count > 0, FP8_ERR_SIZE for
 * count < 0.
 */
typedef struct {
  const void* x;   /* device input, 16-byte aligned */
  int64_t n;       /* elements, >= 0 */
  int32_t dtype;   /* fp8_dtype_t */
  int32_t fmt;     /* fp8_format_t */
  int32_t margin;  /* |margin| <= FP8_MAX_MARGIN */
  int32_t pad;     /* unused */
  uint8_t* y;      /* device, n codes, 16-byte aligned */
  float* amax;     /* device, one float, 4-byte aligned */
  int32_t* bias;   /* device, one int32, 4-byte aligned */
} fp8_quant_desc_t;
int fp8_quantize_multi(const fp8_quant_desc_t* descs, int32_t count, void* stream);

/*
 * The three FP8 x FP8 products with fp32 accumulation, unscaled after the
 * matmul ("Proposed method", bullets 3 and 5).  Each output is overwritten
 * (no accumulation into it).  Operands may be E4M3 or E5M2 in any pairing
 * (E3M4: FP8_ERR_FORMAT).
 * All pointers are device memory; byte operands and outputs must be 16-byte
 * aligned.  M, N, K >= 0 (K == 0 writes zeros; M == 0 or N == 0 is a no-op);
 * FP8_ERR_SIZE for a dimension above 2^31 - 1 or an output of more than
 * 2^31 - 1 tiles of 128 x 128.
 * bx, bw, bdy: device, one int32 each, 4-byte aligned -- the operands'
 * scaling biases.
 *
 * Arithmetic: every product of two FP8 values is exact in fp32 and the sums
 * are formed with fp32 accuracy (FP8_GEMM_EXACT): the FP8 codes are widened
 * exactly to fp16 (both operands E4M3) or bf16 (an E5M2 operand) in registers
 * and multiplied on the 16-bit MFMA, whose products are summed with a 24-bit
 * window.  The native FP8 MFMA of gfx950 is
 * twice as fast but keeps only about 13 bits below the largest of the 64
 * products each instruction sums (an error near 1e-4 of sum|a||b| per
 * instruction); it is available through fp8_scaled_gemm with
 * FP8_GEMM_NATIVE_FP8.
 */
#define FP8_GEMM_EXACT 0      /* fp32-accurate sums (what the three named entry points use) */
#define FP8_GEMM_NATIVE_FP8 1 /* native FP8 MFMA: ~2x faster, ~1e-4 relative per 64 products */

typedef enum {
  FP8_GEMM_FWD = 0,   /* a = X8[M x K],  b = W8[N x K], out = Y[M x N]  */
  FP8_GEMM_DGRAD = 1, /* a = dY8[M x N], b = W8[N x K], out = dX[M x K] */
  FP8_GEMM_WGRAD = 2  /* a = dY8[M x N], b = X8[M x K], out = dW[N x K] */
} fp8_gemm_op_t;

/* Any of the three products with a chosen arithmetic (FP8_GEMM_EXACT or
 * FP8_GEMM_NATIVE_FP8); the named entry points below are this call with
 * FP8_GEMM_EXACT.  Returns FP8_ERR_OP for an unknown op or math.
 * Forward products of few rows (a small batch of tokens through a weight;
 * exact arithmetic, 16-byte aligned rows) run on kernels that stream the
 * weight's rows: 1 to 64 rows with K a multiple of 256 on the exact MFMA
 * (the weight's rows through LDS in 256-byte runs), one or two rows with K
 * another multiple of 16 and M * K <= 65536 on the vector ALU (exact fp32
 * products).  Their results meet the same bound, with the same bits on every
 * call. */
int fp8_scaled_gemm(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                    const int32_t* ba, const uint8_t* b, fp8_format_t fb, const int32_t* bb,
                    int64_t M, int64_t N, int64_t K, float* out, void* stream);

/*
 * Products whose output has too few 128 x 128 tiles to occupy the chip (a
 * small batch of tokens; an output with a short side) run faster split along
 * the contraction: each slice's sum goes to a caller-provided workspace, then
 * the slices are added in slice order and unscaled once, so equal inputs give
 * equal bits on every call.  The number of slices is the cheaper of two:
 * as many as leave one 128 x 128 workgroup per CU beside the output's tiles,
 * or as many as leave two (each slice at least 24 stages of 64 contraction
 * bytes).  These two entry points are for callers who can provide that
 * workspace; fp8_scaled_gemm never splits.
 *
 * fp8_scaled_gemm_workspace_bytes: the workspace bytes fp8_scaled_gemm_ws
 * needs for this product and shape (0: it is not split and needs none), or
 * FP8_ERR_SIZE / FP8_ERR_OP for a bad size or op.  A pure function of
 * (op, M, N, K); no device is touched.
 *
 * fp8_scaled_gemm_ws: fp8_scaled_gemm with a workspace.
 *   ws        device, 16-byte aligned, at least
 *             fp8_scaled_gemm_workspace_bytes(op, M, N, K) bytes (the
 *             caller's; the call overwrites it and keeps no pointer), not
 *             overlapping the operands or the output.  May be NULL when that
 *             is 0.  Calls in flight at the same time need separate
 *             workspaces.
 *   ws_bytes  its size.
 * Returns FP8_ERR_NULL / FP8_ERR_ALIGN / FP8_ERR_SIZE for a missing,
 * misaligned or too small workspace the product needs, otherwise as
 * fp8_scaled_gemm.  Results are within the same bound as fp8_scaled_gemm's
 * (the sums are formed in another order, so the bits may differ from its
 * bits); an unsplit product is fp8_scaled_gemm itself.
 */
int64_t fp8_scaled_gemm_workspace_bytes(fp8_gemm_op_t op, int64_t M, int64_t N, int64_t K);
int fp8_scaled_gemm_ws(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                       const int32_t* ba, const uint8_t* b, fp8_format_t fb, const int32_t* bb,
                       int64_t M, int64_t N, int64_t K, float* out, void* ws, int64_t ws_bytes,
                       void* stream);

/*
 * fp8_scaled_gemm_noalloc: fp8_scaled_gemm_ws for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The split workspace is the library's own static device
 * array of FP8_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, created with the code
 * object and held until the process ends; the call allocates and frees
 * nothing.  Its split takes the plan of fp8_scaled_gemm_ws where that fits
 * the array, and otherwise the one-workgroup-per-CU split, which with the
 * default FP8LIN_SPLIT_SLOTS always fits (at most 256 / tiles slices of an
 * output of tiles 128 x 128 tiles).  Arguments and results are those of
 * fp8_scaled_gemm_ws (the same bits where the plans agree; else within the
 * same bound); a product whose split would still need more scratch than the
 * maximum returns FP8_ERR_SIZE before anything runs.  The first call on a
 * device looks up that device's copy of the array (FP8_ERR_HIP if that
 * fails).
 * Every call on one GPU shares its one array and leaves its contents behind
 * (nothing in it needs clearing: a split product writes every workspace
 * element it reads).  Calls that overlap in time on one GPU -- from two
 * streams, or two host threads -- race on it and corrupt each other's
 * results; callers must order them (one stream, or events).
 */
#define FP8_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int fp8_scaled_gemm_noalloc(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                            const int32_t* ba, const uint8_t* b, fp8_format_t fb,
                            const int32_t* bb, int64_t M, int64_t N, int64_t K, float* out,
                            void* stream);

/*
 * Several products in one call ("Proposed method", bullets 3 and 5: a layer's
 * forward, data-gradient and weight-gradient products), for steps made of
 * many small products, where a launch per product leaves most of the chip
 * idle and pays a dispatch each.  The products of one operand layout and
 * format pair run in one launch (128 x 128 output tiles of all of them);
 * products with long contractions are split into slices of about the
 * shortest contraction among them (raw sums in the workspace, then one
 * launch adds every split product's slices in slice order and unscales), so
 * the launch's blocks do similar work.  Products of 1024 tiles of 128 x 128
 * or more (a whole wave of the single product's 256 x 256 tiles), forward
 * products of few rows through a weight of 16 MiB or more that the small-row
 * kernels take (see fp8_scaled_gemm), or products the pipelined kernels do not
 * take (a contraction that is not a multiple of 64, misaligned rows), run as
 * single products.
 *   descs  host array of count product descriptors (read during the call
 *          only): op and the operands, biases, sizes and output exactly as
 *          fp8_scaled_gemm's arguments.  Outputs must not overlap each other,
 *          any operand or the workspace.
 *   count  0 .. 256.
 *   math   FP8_GEMM_EXACT or FP8_GEMM_NATIVE_FP8, for every product.
 * Every product's output is within the bound of fp8_scaled_gemm's (the same
 * arithmetic; a split one sums in another order), and the same inputs give
 * the same bits on every call.
 *
 * fp8_scaled_gemm_group_workspace_bytes: the workspace bytes the call needs
 * (0: no product is split), a pure function of the descriptors' ops, formats,
 * sizes and alignments, or a negative status (the first bad descriptor's, as
 * fp8_scaled_gemm would return it; FP8_ERR_SIZE for count outside 0 .. 256).
 *
 * fp8_scaled_gemm_group: every argument is checked before anything runs (the
 * first bad descriptor's status; FP8_ERR_NULL / FP8_ERR_ALIGN / FP8_ERR_SIZE
 * for a missing, misaligned or too small workspace the products need).  ws:
 * device, 16-byte aligned, at least the bytes above, the caller's (the call
 * overwrites it and keeps no pointer); calls in flight at the same time need
 * separate workspaces.
 */
typedef struct {
  int32_t op;          /* fp8_gemm_op_t */
  int32_t fa;          /* fp8_format_t of a */
  int32_t fb;          /* fp8_format_t of b */
  int32_t pad;         /* unused */
  const uint8_t* a;    /* device codes, as fp8_scaled_gemm's a */
  const int32_t* ba;   /* device, one int32 */
  const uint8_t* b;    /* device codes, as fp8_scaled_gemm's b */
  const int32_t* bb;   /* device, one int32 */
  int64_t M, N, K;     /* as fp8_scaled_gemm's */
  float* out;          /* device fp32 output */
} fp8_gemm_desc_t;
int64_t fp8_scaled_gemm_group_workspace_bytes(int math, const fp8_gemm_desc_t* descs, int32_t count);
int fp8_scaled_gemm_group(int math, const fp8_gemm_desc_t* descs, int32_t count, void* ws,
                          int64_t ws_bytes, void* stream);

/* fp8_scaled_gemm that also returns the per-tensor amax of its output (the
 * "Proposed method" bullet-1 statistic of the tensor the product produces),
 * computed in the product's own epilogue, so that quantising the output next
 * needs no separate amax pass over it (fp8_compute_bias takes it directly).
 *   out_amax  device, one float, 4-byte aligned, written: max |out| over all
 *             written outputs (0 when there are none; NaN if an output is
 *             NaN), bit-identical to fp8_amax over the fp32 output.
 * Launches a one-lane clear of out_amax, then the product.  Returns
 * FP8_ERR_NULL / FP8_ERR_ALIGN for a null or misaligned out_amax, otherwise
 * as fp8_scaled_gemm. */
int fp8_scaled_gemm_amax(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                         const int32_t* ba, const uint8_t* b, fp8_format_t fb,
                         const int32_t* bb, int64_t M, int64_t N, int64_t K, float* out,
                         float* out_amax, void* stream);

/* fp8_scaled_gemm that adds its result to the output instead of overwriting
 * it: out[i][j] = out[i][j] + 2^-(ba+bb) * sum_k a.b, one fp32
 * round-to-nearest-even addition per output of the sum fp8_scaled_gemm
 * would have stored.  For a weight gradient summed over micro-batches into
 * one fp32 buffer (training, "Proposed method" bullet 5; the pages give the
 * product only as "matmul, then unscale", bullet 3, and accumulating into an
 * existing buffer is this library's reading of the training loop).
 *   out  device, read and written, 16-byte aligned, not overlapping the
 *        operands; calls that overlap in time on one output race.
 * K == 0 adds zero to every output (-0 becomes +0).  Never split along the
 * contraction.  Same checks and status codes as fp8_scaled_gemm.  Within
 * fp8_scaled_gemm's bound plus the addition's own rounding: |out - (old +
 * exact)| <= 1e-5 * 2^-(ba+bb) * sum|a||b| + 2^-24 * |old + exact|. */
int fp8_scaled_gemm_accumulate(fp8_gemm_op_t op, int math, const uint8_t* a, fp8_format_t fa,
                               const int32_t* ba, const uint8_t* b, fp8_format_t fb,
                               const int32_t* bb, int64_t M, int64_t N, int64_t K, float* out,
                               void* stream);

/*
 * The gated activation between the two products of a chained FP8 MLP: Llama
 * 2's SwiGLU (the review page trains Llama 2 models, "Main findings", without
 * naming the activation).  The up-projection is one fused product whose
 * output h [rows x 2f] (fp32, row-major) holds the gate columns g then the up
 * columns u of each row.  With sigmoid(g) = 1 / (1 + e^-g), evaluated in fp32:
 *   fp8_swiglu_fwd:  a[t][j] = g * sigmoid(g) * u                 a: rows x f
 *   fp8_swiglu_bwd:  dh[t][j]     = da * u * sigmoid(g) * (1 + g * (1 - sigmoid(g)))
 *                    dh[t][f + j] = da * g * sigmoid(g)           dh: rows x 2f
 * (g = h[t][j], u = h[t][f + j], da = da[t][j]).  Outputs are bf16 words,
 * rounded to nearest even from the fp32 result (within one bf16 unit in the
 * last place of the exact value, up to fp32 rounding near a midpoint).
 * Non-finite inputs follow IEEE arithmetic of these formulas (g = -inf gives
 * NaN).
 *   out_amax  device float, optional (NULL: not computed), 4-byte aligned:
 *             written with max |output| over the whole output, bit-identical
 *             to fp8_amax over it, so fp8_compute_bias can follow directly
 *             ("Proposed method", bullet 1); 0 for an empty output.
 * h, da, a, dh: device, 16-byte aligned.  rows, f >= 0 (either 0: nothing but
 * the amax clear is launched).  Returns FP8_ERR_SIZE when the launch would need
 * more than 2^31 - 1 blocks: rows * ceil(f / 1024) when f is a multiple of 4,
 * rows * ceil(f / 256) otherwise.
 */
int fp8_swiglu_fwd(const float* h, int64_t rows, int64_t f, uint16_t* a, float* out_amax,
                   void* stream);
int fp8_swiglu_bwd(const float* h, const float* da, int64_t rows, int64_t f, uint16_t* dh,
                   float* out_amax, void* stream);

/* Forward: Y[M x N] = 2^-(bx+bw) * X8[M x K] . W8[N x K]^T */
int fp8_scaled_gemm_fwd(const uint8_t* x8, fp8_format_t fx, const int32_t* bx,
                        const uint8_t* w8, fp8_format_t fw, const int32_t* bw,
                        int64_t M, int64_t N, int64_t K, float* y, void* stream);

/* Data gradient: dX[M x K] = 2^-(bdy+bw) * dY8[M x N] . W8[N x K] */
int fp8_scaled_gemm_dgrad(const uint8_t* dy8, fp8_format_t fdy, const int32_t* bdy,
                          const uint8_t* w8, fp8_format_t fw, const int32_t* bw,
                          int64_t M, int64_t N, int64_t K, float* dx, void* stream);

/* Weight gradient: dW[N x K] = 2^-(bdy+bx) * dY8[M x N]^T . X8[M x K] */
int fp8_scaled_gemm_wgrad(const uint8_t* dy8, fp8_format_t fdy, const int32_t* bdy,
                          const uint8_t* x8, fp8_format_t fx, const int32_t* bx,
                          int64_t M, int64_t N, int64_t K, float* dw, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8LIN_H */
