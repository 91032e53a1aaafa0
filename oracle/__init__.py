"""CPU oracle for the FP8-AMAX scaled linear layer -- TEST INFRASTRUCTURE ONLY.

This package wraps ``oracle.c`` (plain scalar C, compiled with gcc) with ctypes.
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  The HIP library and its Python binding never do,
and this package imports nothing from them.

Method: "Training and inference of large language models using 8-bit floating
point" (Perez, Zhang et al., 2023), review page, section "Proposed method",
bullets 1-4 (per-tensor amax; compute_bias from log2(format max / amplitude)
with a margin; scale before the cast and unscale after the matmul; E4 for
weights and activations, E5 for gradients).  The readings taken where the page
is silent are listed in the header of ``oracle.c``.

Inputs are passed as raw words: bf16 tensors as ``np.uint16``, fp32 tensors as
``np.uint32`` (or ``np.float32``, which is reinterpreted).  FP8 tensors are
``np.uint8`` codes.  Every function here is pinned by ``tests/test_oracle_*``.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16, F32 = 0, 1
E4M3, E5M2, E3M4 = 0, 1, 2
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0, E3M4: 30.0}


def build():
    """Compile oracle.c into liboracle.so next to it (gcc, no fast-math)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)


_lib = None


def lib():
    """The loaded oracle library (built first if nothing is built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64, i32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        L.oracle_threads.restype = ci
        L.oracle_threads.argtypes = []
        L.oracle_amax.restype = ctypes.c_uint32
        L.oracle_amax.argtypes = [vp, ci, i64]
        L.oracle_compute_bias.restype = i32
        L.oracle_compute_bias.argtypes = [ctypes.c_uint32, ci, i32]
        L.oracle_decode_fp8.restype = ctypes.c_double
        L.oracle_decode_fp8.argtypes = [ctypes.c_uint8, ci]
        L.oracle_scale_cast.restype = None
        L.oracle_scale_cast.argtypes = [vp, ci, i64, i32, ci, vp]
        for name in ("oracle_gemm_fwd", "oracle_gemm_dgrad", "oracle_gemm_wgrad"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [vp, ci, i32, vp, ci, i32, i64, i64, i64, vp, vp]
        for name in ("oracle_gemm_fwd_at", "oracle_gemm_dgrad_at", "oracle_gemm_wgrad_at"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [vp, ci, i32, vp, ci, i32, i64, i64, i64, vp, vp, i64, vp, vp]
        L.oracle_swiglu_fwd.restype = None
        L.oracle_swiglu_fwd.argtypes = [vp, i64, i64, vp]
        L.oracle_swiglu_bwd.restype = None
        L.oracle_swiglu_bwd.argtypes = [vp, vp, i64, i64, vp]
        _lib = L
    return _lib


def threads():
    """Threads the oracle's OpenMP loops use."""
    return int(lib().oracle_threads())


def _words(x):
    """(contiguous word array, dtype code) for a bf16-word or fp32 array."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype in (np.uint32, np.float32):
        return x.view(np.uint32), F32
    raise TypeError(f"oracle inputs are bf16 words (uint16) or fp32 words, got {x.dtype}")


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def amax_bits(x):
    """fp32 bit pattern of max|x| (see oracle.c, step 1)."""
    w, dt = _words(x)
    return int(lib().oracle_amax(_ptr(w), dt, w.size))


def amax(x):
    return np.array([amax_bits(x)], dtype=np.uint32).view(np.float32)[0]


def compute_bias(amax_bits_value, fmt, margin=0):
    """floor(log2(fmt_max / amax)) - margin, exactly (see oracle.c, step 2)."""
    return int(lib().oracle_compute_bias(int(amax_bits_value) & 0xFFFFFFFF, int(fmt), int(margin)))


def scale_cast(x, bias, fmt):
    """FP8 codes of x * 2^bias (see oracle.c, step 3)."""
    w, dt = _words(x)
    y = np.empty(w.shape, dtype=np.uint8)
    lib().oracle_scale_cast(_ptr(w), dt, w.size, int(bias), int(fmt), _ptr(y))
    return y


def decode_fp8(codes, fmt):
    """Exact float64 value of each FP8 code."""
    L = lib()
    table = np.array([L.oracle_decode_fp8(c, int(fmt)) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def quantize(x, fmt, margin=0):
    """amax -> bias -> codes, the whole per-tensor quantisation."""
    a = amax_bits(x)
    b = compute_bias(a, fmt, margin)
    return a, b, scale_cast(x, b, fmt)


def _u8(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError("FP8 operands are uint8 code arrays")
    return a


def gemm_fwd(x8, fx, bx, w8, fw, bw):
    """Y = 2^-(bx+bw) * X8 @ W8^T (X8: MxK, W8: NxK).  Returns (Y, bound)."""
    x8, w8 = _u8(x8), _u8(w8)
    (M, K), (N, K2) = x8.shape, w8.shape
    assert K == K2
    y = np.empty((M, N)); bd = np.empty((M, N))
    lib().oracle_gemm_fwd(_ptr(x8), fx, bx, _ptr(w8), fw, bw, M, N, K, _ptr(y), _ptr(bd))
    return y, bd


def gemm_dgrad(dy8, fdy, bdy, w8, fw, bw):
    """dX = 2^-(bdy+bw) * dY8 @ W8 (dY8: MxN, W8: NxK).  Returns (dX, bound)."""
    dy8, w8 = _u8(dy8), _u8(w8)
    (M, N), (N2, K) = dy8.shape, w8.shape
    assert N == N2
    y = np.empty((M, K)); bd = np.empty((M, K))
    lib().oracle_gemm_dgrad(_ptr(dy8), fdy, bdy, _ptr(w8), fw, bw, M, N, K, _ptr(y), _ptr(bd))
    return y, bd


def gemm_wgrad(dy8, fdy, bdy, x8, fx, bx):
    """dW = 2^-(bdy+bx) * dY8^T @ X8 (dY8: MxN, X8: MxK).  Returns (dW, bound)."""
    dy8, x8 = _u8(dy8), _u8(x8)
    (M, N), (M2, K) = dy8.shape, x8.shape
    assert M == M2
    y = np.empty((N, K)); bd = np.empty((N, K))
    lib().oracle_gemm_wgrad(_ptr(dy8), fdy, bdy, _ptr(x8), fx, bx, M, N, K, _ptr(y), _ptr(bd))
    return y, bd


def gemm_accumulate(op, old, a8, fa, ba, b8, fb, bb):
    """old + the product, in float64: the reading that accumulating into an
    existing fp32 buffer (a weight gradient summed over micro-batches, the
    training of "Proposed method" bullet 5) adds the unscaled product of
    bullet 3 to what the buffer holds.  op: 0 fwd, 1 dgrad, 2 wgrad (a, b as
    gemm_fwd / gemm_dgrad / gemm_wgrad take them); old: float32 array of the
    output's shape.  Returns (old + product, the product's bound)."""
    y, bd = (gemm_fwd, gemm_dgrad, gemm_wgrad)[op](a8, fa, ba, b8, fb, bb)
    old = np.asarray(old)
    if old.dtype != np.float32 or old.shape != y.shape:
        raise ValueError(f"old must be float32 of the output's shape {y.shape}")
    return old.astype(np.float64) + y, bd


def _at(fn, a, fa, ba, b, fb, bb, M, N, K, rows, cols):
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(rows.size); bd = np.empty(rows.size)
    fn(_ptr(a), fa, ba, _ptr(b), fb, bb, M, N, K, _ptr(rows), _ptr(cols), rows.size, _ptr(out), _ptr(bd))
    return out, bd


def gemm_fwd_at(x8, fx, bx, w8, fw, bw, rows, cols):
    """Y[rows[t], cols[t]] and its bound, for each t."""
    x8, w8 = _u8(x8), _u8(w8)
    (M, K), (N, _) = x8.shape, w8.shape
    return _at(lib().oracle_gemm_fwd_at, x8, fx, bx, w8, fw, bw, M, N, K, rows, cols)


def gemm_dgrad_at(dy8, fdy, bdy, w8, fw, bw, rows, cols):
    """dX[rows[t], cols[t]] and its bound, for each t."""
    dy8, w8 = _u8(dy8), _u8(w8)
    (M, N), (_, K) = dy8.shape, w8.shape
    return _at(lib().oracle_gemm_dgrad_at, dy8, fdy, bdy, w8, fw, bw, M, N, K, rows, cols)


def gemm_wgrad_at(dy8, fdy, bdy, x8, fx, bx, rows, cols):
    """dW[rows[t], cols[t]] and its bound, for each t."""
    dy8, x8 = _u8(dy8), _u8(x8)
    (M, N), (_, K) = dy8.shape, x8.shape
    return _at(lib().oracle_gemm_wgrad_at, dy8, fdy, bdy, x8, fx, bx, M, N, K, rows, cols)


def _f32(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError("SwiGLU inputs are float32 arrays")
    return a


def swiglu_fwd(h):
    """a = silu(g) * u in float64, h = [g | u] of shape (rows, 2f) (oracle.c, step 5)."""
    h = _f32(h)
    rows, f2 = h.shape
    assert f2 % 2 == 0
    a = np.empty((rows, f2 // 2))
    lib().oracle_swiglu_fwd(_ptr(h), rows, f2 // 2, _ptr(a))
    return a


def swiglu_bwd(h, da):
    """dh = [da * u * silu'(g) | da * silu(g)] in float64 (oracle.c, step 5)."""
    h, da = _f32(h), _f32(da)
    rows, f2 = h.shape
    assert f2 % 2 == 0 and da.shape == (rows, f2 // 2)
    dh = np.empty((rows, f2))
    lib().oracle_swiglu_bwd(_ptr(h), _ptr(da), rows, f2 // 2, _ptr(dh))
    return dh
