"""Python binding of libfp8lin, the FP8-AMAX scaled linear layer for MI355X.

Argument marshalling only: every step runs in the library's HIP kernels
(declared in include/fp8lin.h).  PyTorch provides device memory and the
current stream; results stay on the device.

The method: "Training and inference of large language models using 8-bit
floating point" (Perez, Zhang et al., 2023), review page, "Proposed method":
per-tensor amax -> compute_bias -> scale and cast to E4M3 (weights,
activations) or E5M2 (gradients) -> FP8 matmul, unscaled afterwards.

Layers built on these calls: ``fp8_precision_linear_amd.linear`` (FP8Linear,
the layer with current or delayed scaling) and ``fp8_precision_linear_amd.mlp``
(the chained FP8 MLP with SwiGLU).

Importing this module loads the library and raises ImportError if it is not
built; build it with ``python fp8_precision_linear_amd/build.py``.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8lin.so")

# E3M4: quantisation only (no product takes it).
E4M3, E5M2, E3M4 = 0, 1, 2
BF16, FP32 = 0, 1
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0, E3M4: 30.0}
MAX_MARGIN = 64
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024   # FP8_NOALLOC_SCRATCH_BYTES

STATUS = {0: "FP8_OK", -1: "FP8_ERR_NULL", -2: "FP8_ERR_SIZE", -3: "FP8_ERR_FORMAT",
          -4: "FP8_ERR_DTYPE", -5: "FP8_ERR_ALIGN", -6: "FP8_ERR_MARGIN",
          -7: "FP8_ERR_DEVICE", -8: "FP8_ERR_HIP", -9: "FP8_ERR_OP"}

# Product arithmetic (fp8_scaled_gemm's `math`) and products (its `op`).
MATH_EXACT, MATH_NATIVE_FP8 = 0, 1
OP_FWD, OP_DGRAD, OP_WGRAD = 0, 1, 2

# Exported symbols and their C signatures (include/fp8lin.h).
_vp, _i64, _i32, _ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
SIGNATURES = {
    "fp8_status_string": (ctypes.c_char_p, [_ci]),
    "fp8_amax": (_ci, [_vp, _ci, _i64, _vp, _vp]),
    "fp8_compute_bias": (_ci, [_vp, _ci, _i32, _vp, _vp]),
    "fp8_scale_cast": (_ci, [_vp, _ci, _i64, _vp, _ci, _vp, _vp]),
    "fp8_scale_cast_amax": (_ci, [_vp, _ci, _i64, _vp, _ci, _vp, _vp, _vp]),
    "fp8_quantize": (_ci, [_vp, _ci, _i64, _ci, _i32, _vp, _vp, _vp, _vp]),
    "fp8_quantize_multi": (_ci, [_vp, _i32, _vp]),
    "fp8_quantize_delayed": (_ci, [_vp, _ci, _i64, _ci, _i32, _vp, _vp, _vp, _vp]),
    "fp8_scaled_gemm": (_ci, [_ci, _ci, _vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_amax": (_ci, [_ci, _ci, _vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "fp8_scaled_gemm_accumulate": (_ci, [_ci, _ci, _vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_workspace_bytes": (_i64, [_ci, _i64, _i64, _i64]),
    "fp8_scaled_gemm_ws": (_ci, [_ci, _ci, _vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp]),
    "fp8_scaled_gemm_noalloc": (_ci, [_ci, _ci, _vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_group_workspace_bytes": (_i64, [_ci, _vp, _i32]),
    "fp8_scaled_gemm_group": (_ci, [_ci, _vp, _i32, _vp, _i64, _vp]),
    "fp8_scaled_gemm_fwd": (_ci, [_vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_dgrad": (_ci, [_vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_wgrad": (_ci, [_vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_swiglu_fwd": (_ci, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "fp8_swiglu_bwd": (_ci, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
}


class QuantDesc(ctypes.Structure):
    """fp8_quant_desc_t (include/fp8lin.h): one tensor of fp8_quantize_multi."""
    _fields_ = [("x", ctypes.c_void_p), ("n", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("fmt", ctypes.c_int32), ("margin", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("y", ctypes.c_void_p), ("amax", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class GemmDesc(ctypes.Structure):
    """fp8_gemm_desc_t (include/fp8lin.h): one product of fp8_scaled_gemm_group."""
    _fields_ = [("op", ctypes.c_int32), ("fa", ctypes.c_int32), ("fb", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("a", ctypes.c_void_p), ("ba", ctypes.c_void_p),
                ("b", ctypes.c_void_p), ("bb", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("out", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run python fp8_precision_linear_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


class Fp8Error(RuntimeError):
    def __init__(self, fn, status):
        msg = lib.fp8_status_string(status).decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


def _check(fn, status):
    if status != 0:
        raise Fp8Error(fn, status)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"inputs are bfloat16 or float32 tensors, got {t.dtype}")


def _need_kind(t, name, dtype, numel=None, shape=None):
    """A tensor of `dtype` and, when given, that element count or shape."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_place(t, name, device):
    """A contiguous device tensor on `device`."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA (HIP) tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the operands on {device}")


def _need(t, name, dtype, device, numel=None, shape=None):
    """Check a tensor the library reads or writes before any call (its kind,
    then its place).  A wrong one would otherwise make a kernel write past its
    buffer or to a host address."""
    _need_kind(t, name, dtype, numel, shape)
    _need_place(t, name, device)


def _empty(shape, dtype, device, stream):
    """A new device tensor for a call enqueued on `stream`: allocated on that
    stream, so that torch's caching allocator does not hand its block to
    work on another stream while the call may still use it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _scalar(t, name, dtype, device):
    _need(t, name, dtype, device, numel=1)


def _codes_kind(t, name):
    """FP8 codes: a 2-D uint8 tensor."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D uint8 tensor of FP8 codes")
    _need_kind(t, name, torch.uint8)


def _input(x):
    """A bf16 or fp32 input tensor: its dtype code (TypeError otherwise)."""
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"x must be a tensor, got {type(x).__name__}")
    return _dtype_code(x)


def _places(dev, *named):
    for t, name in named:
        if t is not None:
            _need_place(t, name, dev)


def amax(x, out=None, stream=None):
    """float32[1] device tensor holding max|x| (fp8_amax)."""
    dt = _input(x)
    if out is not None:
        _need_kind(out, "out", torch.float32, numel=1)
    _places(x.device, (x, "x"), (out, "out"))
    out = _empty(1, torch.float32, x.device, stream) if out is None else out
    _check("fp8_amax", lib.fp8_amax(_ptr(x), dt, x.numel(), _ptr(out), _stream(stream)))
    return out


def compute_bias(amax_t, fmt, margin=0, out=None, stream=None):
    """int32[1] device tensor: floor(log2(fmt_max / amax)) - margin (fp8_compute_bias)."""
    _need_kind(amax_t, "amax", torch.float32, numel=1)
    if out is not None:
        _need_kind(out, "out", torch.int32, numel=1)
    _places(amax_t.device, (amax_t, "amax"), (out, "out"))
    out = _empty(1, torch.int32, amax_t.device, stream) if out is None else out
    _check("fp8_compute_bias",
           lib.fp8_compute_bias(_ptr(amax_t), int(fmt), int(margin), _ptr(out), _stream(stream)))
    return out


def scale_cast(x, bias, fmt, out=None, stream=None, amax=None):
    """uint8 device tensor of FP8 codes of x * 2^bias, same shape as x (fp8_scale_cast).
    amax: optional float32[1] device tensor that receives max |x|, folded in the
    same pass (fp8_scale_cast_amax; for delayed scaling)."""
    dt = _input(x)
    _need_kind(bias, "bias", torch.int32, numel=1)
    if out is not None:
        _need_kind(out, "out", torch.uint8, numel=x.numel())
    if amax is not None:
        _need_kind(amax, "amax", torch.float32, numel=1)
    _places(x.device, (x, "x"), (bias, "bias"), (out, "out"), (amax, "amax"))
    out = _empty(x.shape, torch.uint8, x.device, stream) if out is None else out
    if amax is None:
        _check("fp8_scale_cast", lib.fp8_scale_cast(_ptr(x), dt, x.numel(), _ptr(bias),
                                                    int(fmt), _ptr(out), _stream(stream)))
    else:
        _check("fp8_scale_cast_amax",
               lib.fp8_scale_cast_amax(_ptr(x), dt, x.numel(), _ptr(bias), int(fmt),
                                       _ptr(out), _ptr(amax), _stream(stream)))
    return out


def quantize(x, fmt, margin=0, out=None, bias=None, amax=None, stream=None):
    """(codes, bias, amax) of a tensor in one call (fp8_quantize): the results of
    amax -> compute_bias -> scale_cast, in one launch for small tensors and three
    for large ones.  out / bias / amax: optional preallocated device tensors."""
    dt = _input(x)
    if out is not None:
        _need_kind(out, "out", torch.uint8, numel=x.numel())
    if bias is not None:
        _need_kind(bias, "bias", torch.int32, numel=1)
    if amax is not None:
        _need_kind(amax, "amax", torch.float32, numel=1)
    _places(x.device, (x, "x"), (out, "out"), (bias, "bias"), (amax, "amax"))
    out = _empty(x.shape, torch.uint8, x.device, stream) if out is None else out
    bias = _empty(1, torch.int32, x.device, stream) if bias is None else bias
    amax = _empty(1, torch.float32, x.device, stream) if amax is None else amax
    _check("fp8_quantize", lib.fp8_quantize(_ptr(x), dt, x.numel(), int(fmt), int(margin),
                                            _ptr(out), _ptr(amax), _ptr(bias), _stream(stream)))
    return out, bias, amax


def quantize_delayed(x, fmt, amax, margin=0, out=None, bias=None, stream=None):
    """Delayed scaling in one call (fp8_quantize_delayed): the bias from the
    amax the previous step left in `amax` (float32[1] device tensor), the codes
    at that bias, then max |x| of this input into `amax` for the next step.
    Returns (codes, bias); out / bias: optional preallocated device tensors."""
    dt = _input(x)
    _need_kind(amax, "amax", torch.float32, numel=1)
    if out is not None:
        _need_kind(out, "out", torch.uint8, numel=x.numel())
    if bias is not None:
        _need_kind(bias, "bias", torch.int32, numel=1)
    _places(x.device, (x, "x"), (amax, "amax"), (out, "out"), (bias, "bias"))
    out = _empty(x.shape, torch.uint8, x.device, stream) if out is None else out
    bias = _empty(1, torch.int32, x.device, stream) if bias is None else bias
    _check("fp8_quantize_delayed",
           lib.fp8_quantize_delayed(_ptr(x), dt, x.numel(), int(fmt), int(margin), _ptr(out),
                                    _ptr(amax), _ptr(bias), _stream(stream)))
    return out, bias


class QuantizeMulti:
    """fp8_quantize_multi prepared once for fixed tensors: xs and their
    formats and margins; outs (list of (codes, bias, amax)) given or
    allocated here.  run() is then one library call (the tensors' contents
    may change between calls, not their storage)."""

    def __init__(self, xs, fmts, margins=0, outs=None, stream=None):
        xs = list(xs)
        k = len(xs)
        fmts = list(fmts) if isinstance(fmts, (list, tuple)) else [fmts] * k
        margins = list(margins) if isinstance(margins, (list, tuple)) else [margins] * k
        if len(fmts) != k or len(margins) != k or (outs is not None and len(outs) != k):
            raise ValueError("one format, margin and output triple per tensor")
        self.descs = (QuantDesc * max(k, 1))()
        self.outs, self._keep = [], xs
        dev = xs[0].device if k else None
        for i, x in enumerate(xs):
            dt = _input(x)
            if outs is not None:
                out, bias, amax = outs[i]
                _need_kind(out, f"outs[{i}][0]", torch.uint8, numel=x.numel())
                _need_kind(bias, f"outs[{i}][1]", torch.int32, numel=1)
                _need_kind(amax, f"outs[{i}][2]", torch.float32, numel=1)
                _places(dev, (x, f"xs[{i}]"), (out, f"outs[{i}][0]"), (bias, f"outs[{i}][1]"),
                        (amax, f"outs[{i}][2]"))
            else:
                _places(dev, (x, f"xs[{i}]"))
                out = _empty(x.shape, torch.uint8, dev, stream)
                bias = _empty(1, torch.int32, dev, stream)
                amax = _empty(1, torch.float32, dev, stream)
            self.descs[i] = QuantDesc(x.data_ptr(), x.numel(), dt, int(fmts[i]), int(margins[i]), 0,
                                      out.data_ptr(), amax.data_ptr(), bias.data_ptr())
            self.outs.append((out, bias, amax))
        self.count = k
        self.ptr = ctypes.cast(self.descs, ctypes.c_void_p)

    def run(self, stream=None):
        _check("fp8_quantize_multi", lib.fp8_quantize_multi(self.ptr, self.count, _stream(stream)))
        return self.outs


def quantize_multi(xs, fmts, margins=0, outs=None, stream=None):
    """fp8_quantize of every tensor in xs in one call (fp8_quantize_multi: one
    launch per 32 tensors of at most 256 KiB, three per 32 others).  fmts,
    margins: one per tensor, or one for all.  outs: optional list of (codes,
    bias, amax) device tensors to write.  Returns the list of (codes, bias,
    amax), each bit-identical to quantize() of that tensor alone."""
    return QuantizeMulti(xs, fmts, margins, outs=outs, stream=stream).run(stream)


def quantize_chain(x, fmt, margin=0, stream=None):
    """(codes, bias, amax) of a tensor through the three separate calls in order."""
    a = amax(x, stream=stream)
    b = compute_bias(a, fmt, margin, stream=stream)
    return scale_cast(x, b, fmt, stream=stream), b, a


def _gemm_args(op, a8, ba, b8, bb, out, stream):
    """(M, N, K, out) of a product after checking its operands: 2-D uint8
    codes on one device with matching contraction sizes, int32[1] biases, and
    a float32 output of the product's shape (allocated on `stream` if None)."""
    _codes_kind(a8, "a8")
    _codes_kind(b8, "b8")
    _need_kind(ba, "bias_a", torch.int32, numel=1)
    _need_kind(bb, "bias_b", torch.int32, numel=1)
    dev = a8.device
    if op == OP_FWD:                  # X8[M, K], W8[N, K] -> Y[M, N]
        (M, K), (N, K2) = a8.shape, b8.shape
        shape, ok = (M, N), K == K2
    elif op == OP_DGRAD:              # dY8[M, N], W8[N, K] -> dX[M, K]
        (M, N), (N2, K) = a8.shape, b8.shape
        shape, ok = (M, K), N == N2
    elif op == OP_WGRAD:              # dY8[M, N], X8[M, K] -> dW[N, K]
        (M, N), (M2, K) = a8.shape, b8.shape
        shape, ok = (N, K), M == M2
    else:
        raise ValueError(f"unknown op {op}")
    if not ok:
        raise ValueError("contraction sizes differ")
    if out is not None:
        _need_kind(out, "out", torch.float32, shape=shape)
    for t, name in ((a8, "a8"), (b8, "b8"), (ba, "bias_a"), (bb, "bias_b"), (out, "out")):
        if t is not None:
            _need_place(t, name, dev)
    out = _empty(shape, torch.float32, dev, stream) if out is None else out
    return M, N, K, out


def scaled_gemm_fwd(x8, fx, bx, w8, fw, bw, out=None, stream=None):
    """Y[M, N] = 2^-(bx+bw) * X8[M, K] @ W8[N, K]^T in float32 (fp8_scaled_gemm_fwd)."""
    M, N, K, out = _gemm_args(OP_FWD, x8, bx, w8, bw, out, stream)
    _check("fp8_scaled_gemm_fwd",
           lib.fp8_scaled_gemm_fwd(_ptr(x8), int(fx), _ptr(bx), _ptr(w8), int(fw), _ptr(bw),
                                   M, N, K, _ptr(out), _stream(stream)))
    return out


def scaled_gemm_dgrad(dy8, fdy, bdy, w8, fw, bw, out=None, stream=None):
    """dX[M, K] = 2^-(bdy+bw) * dY8[M, N] @ W8[N, K] in float32 (fp8_scaled_gemm_dgrad)."""
    M, N, K, out = _gemm_args(OP_DGRAD, dy8, bdy, w8, bw, out, stream)
    _check("fp8_scaled_gemm_dgrad",
           lib.fp8_scaled_gemm_dgrad(_ptr(dy8), int(fdy), _ptr(bdy), _ptr(w8), int(fw), _ptr(bw),
                                     M, N, K, _ptr(out), _stream(stream)))
    return out


def scaled_gemm_wgrad(dy8, fdy, bdy, x8, fx, bx, out=None, stream=None):
    """dW[N, K] = 2^-(bdy+bx) * dY8[M, N]^T @ X8[M, K] in float32 (fp8_scaled_gemm_wgrad)."""
    M, N, K, out = _gemm_args(OP_WGRAD, dy8, bdy, x8, bx, out, stream)
    _check("fp8_scaled_gemm_wgrad",
           lib.fp8_scaled_gemm_wgrad(_ptr(dy8), int(fdy), _ptr(bdy), _ptr(x8), int(fx), _ptr(bx),
                                     M, N, K, _ptr(out), _stream(stream)))
    return out


def gemm_workspace_bytes(op, M, N, K):
    """Workspace bytes scaled_gemm(..., workspace=...) needs for this product
    (0: it is not split along the contraction) (fp8_scaled_gemm_workspace_bytes)."""
    v = lib.fp8_scaled_gemm_workspace_bytes(int(op), int(M), int(N), int(K))
    if v < 0:
        raise Fp8Error("fp8_scaled_gemm_workspace_bytes", v)
    return v


def scaled_gemm(op, a8, fa, ba, b8, fb, bb, math=MATH_EXACT, out=None, stream=None, amax=None,
                workspace=None):
    """Any of the three products with a chosen arithmetic (fp8_scaled_gemm).
    op: OP_FWD (a = X8[M, K], b = W8[N, K]), OP_DGRAD (a = dY8[M, N], b = W8[N, K])
    or OP_WGRAD (a = dY8[M, N], b = X8[M, K]); math: MATH_EXACT or MATH_NATIVE_FP8.
    amax: optional float32[1] device tensor that receives max |out|, computed
    in the product's epilogue (fp8_scaled_gemm_amax).
    workspace: optional device tensor of at least gemm_workspace_bytes(op, M, N, K)
    bytes; with it an output of few tiles is computed split along the
    contraction (fp8_scaled_gemm_ws).  Not combined with amax."""
    M, N, K, out = _gemm_args(op, a8, ba, b8, bb, out, stream)
    if workspace is not None:
        if amax is not None:
            raise ValueError("a workspace and an output amax are not combined")
        if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != a8.device:
            raise ValueError("workspace must be a contiguous CUDA (HIP) tensor on the operands' device")
        nbytes = workspace.numel() * workspace.element_size()
        _check("fp8_scaled_gemm_ws",
               lib.fp8_scaled_gemm_ws(int(op), int(math), _ptr(a8), int(fa), _ptr(ba), _ptr(b8), int(fb),
                                      _ptr(bb), M, N, K, _ptr(out), _ptr(workspace), nbytes,
                                      _stream(stream)))
    elif amax is None:
        _check("fp8_scaled_gemm",
               lib.fp8_scaled_gemm(int(op), int(math), _ptr(a8), int(fa), _ptr(ba), _ptr(b8), int(fb),
                                   _ptr(bb), M, N, K, _ptr(out), _stream(stream)))
    else:
        _scalar(amax, "amax", torch.float32, a8.device)
        _check("fp8_scaled_gemm_amax",
               lib.fp8_scaled_gemm_amax(int(op), int(math), _ptr(a8), int(fa), _ptr(ba), _ptr(b8),
                                        int(fb), _ptr(bb), M, N, K, _ptr(out), _ptr(amax),
                                        _stream(stream)))
    return out


def scaled_gemm_accumulate(op, a8, fa, ba, b8, fb, bb, out, math=MATH_EXACT, stream=None):
    """out += the product (fp8_scaled_gemm_accumulate): one fp32 addition per
    output of what scaled_gemm would store; out is the caller's float32
    buffer of the product's output shape, read and written in place."""
    if out is None:
        raise ValueError("scaled_gemm_accumulate adds into the caller's output: out is required")
    M, N, K, out = _gemm_args(op, a8, ba, b8, bb, out, stream)
    _check("fp8_scaled_gemm_accumulate",
           lib.fp8_scaled_gemm_accumulate(int(op), int(math), _ptr(a8), int(fa), _ptr(ba), _ptr(b8),
                                          int(fb), _ptr(bb), M, N, K, _ptr(out), _stream(stream)))
    return out


def scaled_gemm_noalloc(op, a8, fa, ba, b8, fb, bb, out, math=MATH_EXACT, stream=None):
    """scaled_gemm with its split workspace in the library's static scratch
    (fp8_scaled_gemm_noalloc): nothing is allocated, so the output is the
    caller's.  Calls on one GPU must not overlap in time (they share the
    scratch)."""
    if out is None:
        raise ValueError("scaled_gemm_noalloc writes the caller's output: out is required")
    M, N, K, out = _gemm_args(op, a8, ba, b8, bb, out, stream)
    _check("fp8_scaled_gemm_noalloc",
           lib.fp8_scaled_gemm_noalloc(int(op), int(math), _ptr(a8), int(fa), _ptr(ba), _ptr(b8), int(fb),
                                       _ptr(bb), M, N, K, _ptr(out), _stream(stream)))
    return out


def scaled_gemm_auto(op, a8, fa, ba, b8, fb, bb, math=MATH_EXACT, out=None, stream=None):
    """scaled_gemm with, when the product is split along the contraction (an
    output of too few tiles to fill the GPU), its workspace taken from
    torch's caching allocator (gemm_workspace_bytes decides), on the stream
    the product runs on."""
    M, N, K, out = _gemm_args(op, a8, ba, b8, bb, out, stream)
    nbytes = gemm_workspace_bytes(op, M, N, K)
    ws = _empty(nbytes, torch.uint8, a8.device, stream) if nbytes > 0 else None
    return scaled_gemm(op, a8, fa, ba, b8, fb, bb, math=math, out=out, stream=stream, workspace=ws)


class GemmGroup:
    """Several products run together (fp8_scaled_gemm_group), prepared once:
    products = [(op, a8, fa, ba, b8, fb, bb), ...] with each output given or
    allocated here.  The descriptors and the workspace are made here, so a
    step can call run() with no host work beyond one ctypes call (the
    tensors' contents may change between calls, not their storage)."""

    def __init__(self, products, outs=None, math=MATH_EXACT, stream=None):
        self.math = math
        self.outs, self._keep = [], []
        k = len(products)
        self.descs = (GemmDesc * max(k, 1))()
        for i, (op, a8, fa, ba, b8, fb, bb) in enumerate(products):
            M, N, K, out = _gemm_args(op, a8, ba, b8, bb, None if outs is None else outs[i], stream)
            self.descs[i] = GemmDesc(int(op), int(fa), int(fb), 0, a8.data_ptr(), ba.data_ptr(), b8.data_ptr(),
                                     bb.data_ptr(), M, N, K, out.data_ptr())
            self.outs.append(out)
            self._keep.append((a8, ba, b8, bb))
        self.count = k
        self.ptr = ctypes.cast(self.descs, ctypes.c_void_p)
        nbytes = lib.fp8_scaled_gemm_group_workspace_bytes(int(math), self.ptr, k)
        if nbytes < 0:
            raise Fp8Error("fp8_scaled_gemm_group_workspace_bytes", nbytes)
        dev = products[0][1].device if k else None
        self.ws = _empty(nbytes, torch.uint8, dev, stream) if nbytes > 0 else None
        self.ws_bytes = nbytes

    def run(self, stream=None):
        _check("fp8_scaled_gemm_group",
               lib.fp8_scaled_gemm_group(int(self.math), self.ptr, self.count, _ptr(self.ws), self.ws_bytes,
                                         _stream(stream)))
        return self.outs


def scaled_gemm_group(products, outs=None, math=MATH_EXACT, stream=None):
    """Run several products together once (see GemmGroup); returns their outputs."""
    return GemmGroup(products, outs=outs, math=math, stream=stream).run(stream)


def swiglu_fwd(h, out=None, amax=None, stream=None):
    """a = silu(g) * u as a bf16 tensor [rows, f], h = [g | u] float32 [rows, 2f]
    (fp8_swiglu_fwd).  amax: optional float32[1] device tensor that receives
    max |a|."""
    if not isinstance(h, torch.Tensor) or h.dtype != torch.float32 or h.dim() != 2 or h.shape[1] % 2:
        raise ValueError("h must be a float32 [rows, 2f] tensor")
    rows, f = h.shape[0], h.shape[1] // 2
    if out is not None:
        _need_kind(out, "out", torch.bfloat16, shape=(rows, f))
    if amax is not None:
        _need_kind(amax, "amax", torch.float32, numel=1)
    _places(h.device, (h, "h"), (out, "out"), (amax, "amax"))
    out = _empty((rows, f), torch.bfloat16, h.device, stream) if out is None else out
    _check("fp8_swiglu_fwd", lib.fp8_swiglu_fwd(_ptr(h), rows, f, _ptr(out), _ptr(amax), _stream(stream)))
    return out


def swiglu_bwd(h, da, out=None, amax=None, stream=None):
    """dh = [da * u * silu'(g) | da * silu(g)] as a bf16 tensor [rows, 2f]
    (fp8_swiglu_bwd); da float32 [rows, f].  amax: optional float32[1] device
    tensor that receives max |dh|."""
    if not isinstance(h, torch.Tensor) or h.dtype != torch.float32 or h.dim() != 2 or h.shape[1] % 2:
        raise ValueError("h must be a float32 [rows, 2f] tensor")
    rows, f = h.shape[0], h.shape[1] // 2
    _need_kind(da, "da", torch.float32, shape=(rows, f))
    if out is not None:
        _need_kind(out, "out", torch.bfloat16, shape=(rows, 2 * f))
    if amax is not None:
        _need_kind(amax, "amax", torch.float32, numel=1)
    _places(h.device, (h, "h"), (da, "da"), (out, "out"), (amax, "amax"))
    out = _empty((rows, 2 * f), torch.bfloat16, h.device, stream) if out is None else out
    _check("fp8_swiglu_bwd", lib.fp8_swiglu_bwd(_ptr(h), _ptr(da), rows, f, _ptr(out), _ptr(amax),
                                                _stream(stream)))
    return out
