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
    "fp8_scaled_gemm": (_ci, [_ci, _ci, _vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_amax": (_ci, [_ci, _ci, _vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "fp8_scaled_gemm_workspace_bytes": (_i64, [_ci, _i64, _i64, _i64]),
    "fp8_scaled_gemm_ws": (_ci, [_ci, _ci, _vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp]),
    "fp8_scaled_gemm_noalloc": (_ci, [_ci, _ci, _vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_fwd": (_ci, [_vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_dgrad": (_ci, [_vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_scaled_gemm_wgrad": (_ci, [_vp, _ci, _vp, _vp, _ci, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_swiglu_fwd": (_ci, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "fp8_swiglu_bwd": (_ci, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
}


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


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA (HIP) tensors")


def amax(x, out=None, stream=None):
    """float32[1] device tensor holding max|x| (fp8_amax)."""
    _need_cuda(x)
    out = torch.empty(1, dtype=torch.float32, device=x.device) if out is None else out
    _check("fp8_amax", lib.fp8_amax(_ptr(x), _dtype_code(x), x.numel(), _ptr(out), _stream(stream)))
    return out


def compute_bias(amax_t, fmt, margin=0, out=None, stream=None):
    """int32[1] device tensor: floor(log2(fmt_max / amax)) - margin (fp8_compute_bias)."""
    _need_cuda(amax_t)
    out = torch.empty(1, dtype=torch.int32, device=amax_t.device) if out is None else out
    _check("fp8_compute_bias",
           lib.fp8_compute_bias(_ptr(amax_t), int(fmt), int(margin), _ptr(out), _stream(stream)))
    return out


def scale_cast(x, bias, fmt, out=None, stream=None, amax=None):
    """uint8 device tensor of FP8 codes of x * 2^bias, same shape as x (fp8_scale_cast).
    amax: optional float32[1] device tensor that receives max |x|, folded in the
    same pass (fp8_scale_cast_amax; for delayed scaling)."""
    _need_cuda(x, bias)
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    if amax is None:
        _check("fp8_scale_cast", lib.fp8_scale_cast(_ptr(x), _dtype_code(x), x.numel(), _ptr(bias),
                                                    int(fmt), _ptr(out), _stream(stream)))
    else:
        _need_cuda(amax)
        _check("fp8_scale_cast_amax",
               lib.fp8_scale_cast_amax(_ptr(x), _dtype_code(x), x.numel(), _ptr(bias), int(fmt),
                                       _ptr(out), _ptr(amax), _stream(stream)))
    return out


def quantize(x, fmt, margin=0, out=None, bias=None, amax=None, stream=None):
    """(codes, bias, amax) of a tensor in one call (fp8_quantize): the results of
    amax -> compute_bias -> scale_cast, in one launch for small tensors and three
    for large ones.  out / bias / amax: optional preallocated device tensors."""
    _need_cuda(x)
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    bias = torch.empty(1, dtype=torch.int32, device=x.device) if bias is None else bias
    amax = torch.empty(1, dtype=torch.float32, device=x.device) if amax is None else amax
    _need_cuda(out, bias, amax)
    _check("fp8_quantize", lib.fp8_quantize(_ptr(x), _dtype_code(x), x.numel(), int(fmt), int(margin),
                                            _ptr(out), _ptr(amax), _ptr(bias), _stream(stream)))
    return out, bias, amax


def quantize_chain(x, fmt, margin=0, stream=None):
    """(codes, bias, amax) of a tensor through the three separate calls in order."""
    a = amax(x, stream=stream)
    b = compute_bias(a, fmt, margin, stream=stream)
    return scale_cast(x, b, fmt, stream=stream), b, a


def scaled_gemm_fwd(x8, fx, bx, w8, fw, bw, out=None, stream=None):
    """Y[M, N] = 2^-(bx+bw) * X8[M, K] @ W8[N, K]^T in float32 (fp8_scaled_gemm_fwd)."""
    _need_cuda(x8, w8, bx, bw)
    M, K = x8.shape
    N, K2 = w8.shape
    if K != K2:
        raise ValueError("contraction sizes differ")
    out = torch.empty((M, N), dtype=torch.float32, device=x8.device) if out is None else out
    _check("fp8_scaled_gemm_fwd",
           lib.fp8_scaled_gemm_fwd(_ptr(x8), int(fx), _ptr(bx), _ptr(w8), int(fw), _ptr(bw),
                                   M, N, K, _ptr(out), _stream(stream)))
    return out


def scaled_gemm_dgrad(dy8, fdy, bdy, w8, fw, bw, out=None, stream=None):
    """dX[M, K] = 2^-(bdy+bw) * dY8[M, N] @ W8[N, K] in float32 (fp8_scaled_gemm_dgrad)."""
    _need_cuda(dy8, w8, bdy, bw)
    M, N = dy8.shape
    N2, K = w8.shape
    if N != N2:
        raise ValueError("contraction sizes differ")
    out = torch.empty((M, K), dtype=torch.float32, device=dy8.device) if out is None else out
    _check("fp8_scaled_gemm_dgrad",
           lib.fp8_scaled_gemm_dgrad(_ptr(dy8), int(fdy), _ptr(bdy), _ptr(w8), int(fw), _ptr(bw),
                                     M, N, K, _ptr(out), _stream(stream)))
    return out


def scaled_gemm_wgrad(dy8, fdy, bdy, x8, fx, bx, out=None, stream=None):
    """dW[N, K] = 2^-(bdy+bx) * dY8[M, N]^T @ X8[M, K] in float32 (fp8_scaled_gemm_wgrad)."""
    _need_cuda(dy8, x8, bdy, bx)
    M, N = dy8.shape
    M2, K = x8.shape
    if M != M2:
        raise ValueError("contraction sizes differ")
    out = torch.empty((N, K), dtype=torch.float32, device=dy8.device) if out is None else out
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
    _need_cuda(a8, b8, ba, bb)
    if op == OP_FWD:
        (M, K), (N, K2) = a8.shape, b8.shape
        shape, ok = (M, N), K == K2
    elif op == OP_DGRAD:
        (M, N), (N2, K) = a8.shape, b8.shape
        shape, ok = (M, K), N == N2
    elif op == OP_WGRAD:
        (M, N), (M2, K) = a8.shape, b8.shape
        shape, ok = (N, K), M == M2
    else:
        raise ValueError(f"unknown op {op}")
    if not ok:
        raise ValueError("contraction sizes differ")
    out = torch.empty(shape, dtype=torch.float32, device=a8.device) if out is None else out
    if workspace is not None:
        if amax is not None:
            raise ValueError("a workspace and an output amax are not combined")
        _need_cuda(workspace)
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
        _need_cuda(amax)
        _check("fp8_scaled_gemm_amax",
               lib.fp8_scaled_gemm_amax(int(op), int(math), _ptr(a8), int(fa), _ptr(ba), _ptr(b8),
                                        int(fb), _ptr(bb), M, N, K, _ptr(out), _ptr(amax),
                                        _stream(stream)))
    return out


def scaled_gemm_noalloc(op, a8, fa, ba, b8, fb, bb, out, math=MATH_EXACT, stream=None):
    """scaled_gemm with its split workspace in the library's static scratch
    (fp8_scaled_gemm_noalloc): nothing is allocated, so the output is the
    caller's.  Calls on one GPU must not overlap in time (they share the
    scratch)."""
    _need_cuda(a8, b8, ba, bb, out)
    if op == OP_FWD:                  # X8[M, K], W8[N, K]
        (M, K), N = a8.shape, b8.shape[0]
    else:                             # dY8[M, N] with W8[N, K] (dgrad) or X8[M, K] (wgrad)
        (M, N), K = a8.shape, b8.shape[1]
    _check("fp8_scaled_gemm_noalloc",
           lib.fp8_scaled_gemm_noalloc(int(op), int(math), _ptr(a8), int(fa), _ptr(ba), _ptr(b8), int(fb),
                                       _ptr(bb), M, N, K, _ptr(out), _stream(stream)))
    return out


def scaled_gemm_auto(op, a8, fa, ba, b8, fb, bb, math=MATH_EXACT, out=None, stream=None):
    """scaled_gemm with, when the product is split along the contraction (an
    output of too few tiles to fill the GPU), its workspace taken from
    torch's caching allocator (gemm_workspace_bytes decides)."""
    if op == OP_FWD:                  # X8[M, K], W8[N, K]
        (M, K), N = a8.shape, b8.shape[0]
    else:                             # dY8[M, N] with W8[N, K] (dgrad) or X8[M, K] (wgrad)
        (M, N), K = a8.shape, b8.shape[1]
    nbytes = gemm_workspace_bytes(op, M, N, K)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=a8.device) if nbytes > 0 else None
    return scaled_gemm(op, a8, fa, ba, b8, fb, bb, math=math, out=out, stream=stream, workspace=ws)


def swiglu_fwd(h, out=None, amax=None, stream=None):
    """a = silu(g) * u as a bf16 tensor [rows, f], h = [g | u] float32 [rows, 2f]
    (fp8_swiglu_fwd).  amax: optional float32[1] device tensor that receives
    max |a|."""
    _need_cuda(h)
    if h.dtype != torch.float32 or h.dim() != 2 or h.shape[1] % 2:
        raise ValueError("h must be a float32 [rows, 2f] tensor")
    rows, f = h.shape[0], h.shape[1] // 2
    out = torch.empty((rows, f), dtype=torch.bfloat16, device=h.device) if out is None else out
    _need_cuda(out, amax)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (rows, f):
        raise ValueError("out must be a bfloat16 [rows, f] tensor")
    _check("fp8_swiglu_fwd", lib.fp8_swiglu_fwd(_ptr(h), rows, f, _ptr(out), _ptr(amax), _stream(stream)))
    return out


def swiglu_bwd(h, da, out=None, amax=None, stream=None):
    """dh = [da * u * silu'(g) | da * silu(g)] as a bf16 tensor [rows, 2f]
    (fp8_swiglu_bwd); da float32 [rows, f].  amax: optional float32[1] device
    tensor that receives max |dh|."""
    _need_cuda(h, da)
    if h.dtype != torch.float32 or h.dim() != 2 or h.shape[1] % 2:
        raise ValueError("h must be a float32 [rows, 2f] tensor")
    rows, f = h.shape[0], h.shape[1] // 2
    if da.dtype != torch.float32 or tuple(da.shape) != (rows, f):
        raise ValueError("da must be a float32 [rows, f] tensor")
    out = torch.empty((rows, 2 * f), dtype=torch.bfloat16, device=h.device) if out is None else out
    _need_cuda(out, amax)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (rows, 2 * f):
        raise ValueError("out must be a bfloat16 [rows, 2f] tensor")
    _check("fp8_swiglu_bwd", lib.fp8_swiglu_bwd(_ptr(h), _ptr(da), rows, f, _ptr(out), _ptr(amax),
                                                _stream(stream)))
    return out
