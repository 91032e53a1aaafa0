"""The C ABI without a GPU: the library loads, exports every function that
include/fp8lin.h declares, and rejects bad arguments on the host before any
HIP call, with the documented status codes."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8lin.h")

import fp8_precision_linear_amd as fl  # noqa: E402

L = fl.lib
P = ctypes.c_void_p
A16, A32, A48 = P(16), P(32), P(48)   # aligned fake addresses: never dereferenced here
MIS = P(17)                           # misaligned fake address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)))


def status(code):
    return {v: k for k, v in fl.STATUS.items()}[code]


def test_every_declared_function_is_exported_and_bound():
    names = declared_functions()
    assert len(names) == 21
    for n in names:
        assert hasattr(L, n), n
        assert n in fl.SIGNATURES, n


def test_status_strings():
    for code in list(fl.STATUS) + [-99]:
        s = L.fp8_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0


def test_amax_argument_checks():
    assert L.fp8_amax(A16, 0, -1, A32, None) == status("FP8_ERR_SIZE")
    assert L.fp8_amax(A16, 7, 10, A32, None) == status("FP8_ERR_DTYPE")
    assert L.fp8_amax(None, 0, 10, A32, None) == status("FP8_ERR_NULL")
    assert L.fp8_amax(A16, 0, 10, None, None) == status("FP8_ERR_NULL")
    assert L.fp8_amax(MIS, 1, 10, A32, None) == status("FP8_ERR_ALIGN")
    assert L.fp8_amax(A16, 0, 10, P(18), None) == status("FP8_ERR_ALIGN")   # amax word
    assert L.fp8_amax(None, 0, 0, P(18), None) == status("FP8_ERR_ALIGN")   # also when empty


def test_bias_argument_checks():
    assert L.fp8_compute_bias(A16, 3, 0, A32, None) == status("FP8_ERR_FORMAT")
    assert L.fp8_compute_bias(A16, 0, 65, A32, None) == status("FP8_ERR_MARGIN")
    assert L.fp8_compute_bias(A16, 1, -65, A32, None) == status("FP8_ERR_MARGIN")
    assert L.fp8_compute_bias(None, 0, 0, A32, None) == status("FP8_ERR_NULL")
    assert L.fp8_compute_bias(A16, 0, 0, None, None) == status("FP8_ERR_NULL")
    assert L.fp8_compute_bias(P(18), 0, 0, A32, None) == status("FP8_ERR_ALIGN")
    assert L.fp8_compute_bias(A16, 0, 0, P(34), None) == status("FP8_ERR_ALIGN")


def test_cast_argument_checks():
    assert L.fp8_scale_cast(A16, 0, -5, A32, 0, A48, None) == status("FP8_ERR_SIZE")
    assert L.fp8_scale_cast(A16, 3, 5, A32, 0, A48, None) == status("FP8_ERR_DTYPE")
    assert L.fp8_scale_cast(A16, 0, 5, A32, -1, A48, None) == status("FP8_ERR_FORMAT")
    assert L.fp8_scale_cast(A16, 0, 5, A32, 3, A48, None) == status("FP8_ERR_FORMAT")
    assert L.fp8_scale_cast(A16, 0, 5, None, 0, A48, None) == status("FP8_ERR_NULL")
    assert L.fp8_scale_cast(A16, 0, 5, A32, 0, None, None) == status("FP8_ERR_NULL")
    assert L.fp8_scale_cast(MIS, 0, 5, A32, 0, A48, None) == status("FP8_ERR_ALIGN")
    assert L.fp8_scale_cast(A16, 0, 5, A32, 0, MIS, None) == status("FP8_ERR_ALIGN")
    assert L.fp8_scale_cast(A16, 0, 5, P(33), 0, A48, None) == status("FP8_ERR_ALIGN")   # bias word
    # n == 0 is a no-op: nothing is checked further and nothing is launched
    assert L.fp8_scale_cast(None, 0, 0, None, 0, None, None) == 0


@pytest.mark.parametrize("fn", ["fp8_scaled_gemm_fwd", "fp8_scaled_gemm_dgrad", "fp8_scaled_gemm_wgrad"])
def test_gemm_argument_checks(fn):
    f = getattr(L, fn)
    ok = (A16, 0, A32, A48, 0, A32, 64, 64, 64, A16, None)

    def call(**kw):
        a = list(ok)
        names = ["a", "fa", "ba", "b", "fb", "bb", "M", "N", "K", "out", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(M=-1) == status("FP8_ERR_SIZE")
    assert call(K=1 << 31) == status("FP8_ERR_SIZE")
    # an output of more than 2^31 - 1 tiles of 128 x 128 (each side fits)
    out_rows, out_cols = {"fp8_scaled_gemm_fwd": ("M", "N"), "fp8_scaled_gemm_dgrad": ("M", "K"),
                          "fp8_scaled_gemm_wgrad": ("N", "K")}[fn]
    assert call(**{out_rows: (1 << 31) - 1, out_cols: (1 << 31) - 1}) == status("FP8_ERR_SIZE")
    assert call(fa=2) == status("FP8_ERR_FORMAT")     # E3M4: no product takes it
    assert call(fb=2) == status("FP8_ERR_FORMAT")
    assert call(fa=3) == status("FP8_ERR_FORMAT")
    assert call(fb=-1) == status("FP8_ERR_FORMAT")
    assert call(out=None) == status("FP8_ERR_NULL")
    assert call(ba=None) == status("FP8_ERR_NULL")
    assert call(a=None) == status("FP8_ERR_NULL")
    assert call(b=None) == status("FP8_ERR_NULL")
    assert call(a=MIS) == status("FP8_ERR_ALIGN")
    assert call(out=MIS) == status("FP8_ERR_ALIGN")
    assert call(ba=P(34)) == status("FP8_ERR_ALIGN")
    assert call(bb=P(35)) == status("FP8_ERR_ALIGN")
    # sizes whose element counts overflow int64 are rejected by the range check
    assert call(M=1 << 62, K=1 << 62) == status("FP8_ERR_SIZE")
    # an empty output is a no-op whatever the pointers are; an empty
    # contraction still writes the (zero) output, so it needs the pointers
    out_dim, contraction = {"fp8_scaled_gemm_fwd": ("M", "K"), "fp8_scaled_gemm_dgrad": ("M", "N"),
                            "fp8_scaled_gemm_wgrad": ("N", "M")}[fn]
    assert call(**{out_dim: 0}, a=None, b=None, out=None, ba=None) == 0
    assert call(**{contraction: 0}, out=None) == status("FP8_ERR_NULL")


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_valid_calls_without_a_device_report_no_device():
    assert L.fp8_amax(A16, 0, 10, A32, None) == status("FP8_ERR_DEVICE")
    assert L.fp8_compute_bias(A16, 0, 0, A32, None) == status("FP8_ERR_DEVICE")
    assert L.fp8_scale_cast(A16, 0, 5, A32, 0, A48, None) == status("FP8_ERR_DEVICE")
    assert L.fp8_scaled_gemm_fwd(A16, 0, A32, A48, 0, A32, 64, 64, 64, A16, None) == status("FP8_ERR_DEVICE")


def test_python_wrappers_reject_cpu_tensors():
    x = torch.zeros(16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fl.amax(x)


def _raises(fn, text):
    with pytest.raises(ValueError) as e:
        fn()
    assert text in str(e.value), str(e.value)


def test_python_wrappers_check_outputs_before_calling():
    """Every output, bias and code tensor is checked for dtype and size (then
    for being a contiguous device tensor) before the library is called: a
    wrong one would make a kernel write past its buffer or to a host address."""
    x = torch.zeros(16, dtype=torch.bfloat16)
    i32, f32, u8 = torch.int32, torch.float32, torch.uint8
    one = lambda dt: torch.zeros(1, dtype=dt)
    _raises(lambda: fl.amax(x, out=torch.zeros(1, dtype=torch.bfloat16)), "out must be torch.float32")
    _raises(lambda: fl.amax(x, out=torch.zeros(2, dtype=f32)), "out must hold 1 elements")
    _raises(lambda: fl.compute_bias(one(i32), 0), "amax must be torch.float32")
    _raises(lambda: fl.compute_bias(one(f32), 0, out=one(f32)), "out must be torch.int32")
    _raises(lambda: fl.scale_cast(x, one(f32), 0), "bias must be torch.int32")
    _raises(lambda: fl.scale_cast(x, torch.zeros(2, dtype=i32), 0), "bias must hold 1 elements")
    _raises(lambda: fl.scale_cast(x, one(i32), 0, out=torch.zeros(15, dtype=u8)), "out must hold 16 elements")
    _raises(lambda: fl.scale_cast(x, one(i32), 0, out=torch.zeros(16, dtype=torch.int8)), "out must be torch.uint8")
    _raises(lambda: fl.scale_cast(x, one(i32), 0, amax=one(i32)), "amax must be torch.float32")
    _raises(lambda: fl.quantize(x, 0, out=torch.zeros(8, dtype=u8)), "out must hold 16 elements")
    _raises(lambda: fl.quantize(x, 0, bias=one(f32)), "bias must be torch.int32")
    _raises(lambda: fl.quantize(x, 0, amax=torch.zeros(4, dtype=f32)), "amax must hold 1 elements")
    with pytest.raises(TypeError):
        fl.quantize(torch.zeros(16, dtype=torch.float16), 0)
    a8, b8 = torch.zeros(4, 8, dtype=u8), torch.zeros(6, 8, dtype=u8)
    bi = one(i32)
    _raises(lambda: fl.scaled_gemm(fl.OP_FWD, a8, 0, bi, b8, 0, bi, out=torch.zeros(4, 6, dtype=torch.bfloat16)),
            "out must be torch.float32")
    _raises(lambda: fl.scaled_gemm(fl.OP_FWD, a8, 0, bi, b8, 0, bi, out=torch.zeros(6, 4)), "out must have shape (4, 6)")
    _raises(lambda: fl.scaled_gemm_dgrad(torch.zeros(4, 6, dtype=u8), 1, bi, b8, 0, bi, out=torch.zeros(4, 6)),
            "out must have shape (4, 8)")
    _raises(lambda: fl.scaled_gemm_wgrad(torch.zeros(4, 6, dtype=u8), 1, bi, a8, 0, bi, out=torch.zeros(8, 6)),
            "out must have shape (6, 8)")
    _raises(lambda: fl.scaled_gemm_fwd(a8.to(torch.int8), 0, bi, b8, 0, bi), "a8 must be torch.uint8")
    _raises(lambda: fl.scaled_gemm_fwd(a8, 0, one(f32), b8, 0, bi), "bias_a must be torch.int32")
    _raises(lambda: fl.scaled_gemm_fwd(a8, 0, bi, b8, 0, torch.zeros(2, dtype=i32)), "bias_b must hold 1 elements")
    _raises(lambda: fl.scaled_gemm_fwd(a8.reshape(-1), 0, bi, b8, 0, bi), "2-D uint8")
    _raises(lambda: fl.scaled_gemm_fwd(a8, 0, bi, torch.zeros(6, 7, dtype=u8), 0, bi), "contraction sizes differ")
    _raises(lambda: fl.scaled_gemm_noalloc(fl.OP_FWD, a8, 0, bi, b8, 0, bi, None), "out is required")
    _raises(lambda: fl.scaled_gemm_noalloc(fl.OP_FWD, a8, 0, bi, b8, 0, bi, torch.zeros(4, 6, dtype=torch.float64)),
            "out must be torch.float32")
    # right kinds on the host: refused for not being device tensors
    _raises(lambda: fl.scaled_gemm(fl.OP_FWD, a8, 0, bi, b8, 0, bi, out=torch.zeros(4, 6)), "CUDA (HIP) tensor")
    h = torch.zeros(3, 8)
    _raises(lambda: fl.swiglu_fwd(h, out=torch.zeros(3, 4)), "out must be torch.bfloat16")
    _raises(lambda: fl.swiglu_fwd(h, amax=torch.zeros(1, dtype=torch.bfloat16)), "amax must be torch.float32")
    _raises(lambda: fl.swiglu_bwd(h, torch.zeros(3, 5)), "da must have shape (3, 4)")
    _raises(lambda: fl.swiglu_bwd(h, torch.zeros(3, 4), out=torch.zeros(3, 4, dtype=torch.bfloat16)),
            "out must have shape (3, 8)")


def test_generic_gemm_rejects_unknown_op_and_math():
    assert L.fp8_scaled_gemm(3, 0, A16, 0, A32, A48, 0, A32, 8, 8, 8, A16, None) == status("FP8_ERR_OP")
    assert L.fp8_scaled_gemm(0, 2, A16, 0, A32, A48, 0, A32, 8, 8, 8, A16, None) == status("FP8_ERR_OP")
    assert L.fp8_scaled_gemm(0, -1, A16, 0, A32, A48, 0, A32, 8, 8, 8, A16, None) == status("FP8_ERR_OP")
    for op in (0, 1, 2):
        assert L.fp8_scaled_gemm(op, 1, A16, 5, A32, A48, 0, A32, 8, 8, 8, A16, None) == status("FP8_ERR_FORMAT")
        assert L.fp8_scaled_gemm(op, 0, A16, 0, A32, A48, 0, A32, 8, 8, 8, None, None) == status("FP8_ERR_NULL")


def test_gemm_amax_argument_checks():
    """fp8_scaled_gemm_amax checks its amax output first, then everything
    fp8_scaled_gemm checks, all before any HIP call."""
    f = L.fp8_scaled_gemm_amax
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 8, 8, 8, A16, None, None) == status("FP8_ERR_NULL")
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 8, 8, 8, A16, P(18), None) == status("FP8_ERR_ALIGN")
    assert f(3, 0, A16, 0, A32, A48, 0, A32, 8, 8, 8, A16, A32, None) == status("FP8_ERR_OP")
    assert f(0, 2, A16, 0, A32, A48, 0, A32, 8, 8, 8, A16, A32, None) == status("FP8_ERR_OP")
    for op in (0, 1, 2):
        assert f(op, 0, A16, 7, A32, A48, 0, A32, 8, 8, 8, A16, A32, None) == status("FP8_ERR_FORMAT")
        assert f(op, 0, A16, 0, A32, A48, 0, A32, 8, 8, 8, None, A32, None) == status("FP8_ERR_NULL")
        assert f(op, 0, MIS, 0, A32, A48, 0, A32, 8, 8, 8, A16, A32, None) == status("FP8_ERR_ALIGN")
        assert f(op, 0, A16, 0, A32, A48, 0, A32, -1, 8, 8, A16, A32, None) == status("FP8_ERR_SIZE")


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_gemm_amax_without_a_device_reports_no_device():
    """Even an empty product must clear its amax output, so it needs the device."""
    f = L.fp8_scaled_gemm_amax
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 0, 8, 8, A16, A32, None) == status("FP8_ERR_DEVICE")
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 64, 64, 64, A16, A32, None) == status("FP8_ERR_DEVICE")


def test_gemm_accumulate_argument_checks():
    """fp8_scaled_gemm_accumulate checks what fp8_scaled_gemm checks, before
    any HIP call; an empty output is a no-op."""
    f = L.fp8_scaled_gemm_accumulate
    assert f(3, 0, A16, 0, A32, A48, 0, A32, 8, 8, 8, A16, None) == status("FP8_ERR_OP")
    assert f(0, 2, A16, 0, A32, A48, 0, A32, 8, 8, 8, A16, None) == status("FP8_ERR_OP")
    for op in (0, 1, 2):
        assert f(op, 0, A16, 2, A32, A48, 0, A32, 8, 8, 8, A16, None) == status("FP8_ERR_FORMAT")
        assert f(op, 0, A16, 0, A32, A48, 0, A32, 8, 8, 8, None, None) == status("FP8_ERR_NULL")
        assert f(op, 0, A16, 0, None, A48, 0, A32, 8, 8, 8, A16, None) == status("FP8_ERR_NULL")
        assert f(op, 0, A16, 0, A32, A48, 0, A32, 8, 8, 8, MIS, None) == status("FP8_ERR_ALIGN")
        assert f(op, 0, A16, 0, A32, A48, 0, A32, -1, 8, 8, A16, None) == status("FP8_ERR_SIZE")
    assert f(0, 0, None, 0, None, None, 0, None, 0, 8, 8, None, None) == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_gemm_accumulate_without_a_device_reports_no_device():
    f = L.fp8_scaled_gemm_accumulate
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 64, 64, 64, A16, None) == status("FP8_ERR_DEVICE")


def test_gemm_accumulate_wrapper_needs_an_output():
    a8 = torch.zeros(8, 8, dtype=torch.uint8)
    b0 = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError):
        fl.scaled_gemm_accumulate(fl.OP_FWD, a8, fl.E4M3, b0, a8, fl.E4M3, b0, None)
    with pytest.raises(ValueError):   # CPU tensors
        fl.scaled_gemm_accumulate(fl.OP_FWD, a8, fl.E4M3, b0, a8, fl.E4M3, b0, torch.zeros(8, 8))


def test_swiglu_argument_checks():
    fwd, bwd = L.fp8_swiglu_fwd, L.fp8_swiglu_bwd
    assert fwd(A16, -1, 4, A32, None, None) == status("FP8_ERR_SIZE")
    assert fwd(A16, 4, -4, A32, None, None) == status("FP8_ERR_SIZE")
    assert fwd(A16, 1 << 31, 4, A32, None, None) == status("FP8_ERR_SIZE")
    assert fwd(A16, (1 << 31) - 1, 1 << 29, A32, None, None) == status("FP8_ERR_SIZE")   # grid too large
    assert fwd(None, 4, 4, A32, None, None) == status("FP8_ERR_NULL")
    assert fwd(A16, 4, 4, None, None, None) == status("FP8_ERR_NULL")
    assert fwd(MIS, 4, 4, A32, None, None) == status("FP8_ERR_ALIGN")
    assert fwd(A16, 4, 4, MIS, None, None) == status("FP8_ERR_ALIGN")
    assert fwd(A16, 4, 4, A32, P(18), None) == status("FP8_ERR_ALIGN")
    assert bwd(A16, None, 4, 4, A32, None, None) == status("FP8_ERR_NULL")
    assert bwd(A16, MIS, 4, 4, A32, None, None) == status("FP8_ERR_ALIGN")
    assert bwd(A16, A48, -4, 4, A32, None, None) == status("FP8_ERR_SIZE")
    # empty without an amax: nothing to do, no device needed
    assert fwd(None, 0, 4, None, None, None) == 0
    assert bwd(None, None, 4, 0, None, None, None) == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_swiglu_without_a_device_reports_no_device():
    assert L.fp8_swiglu_fwd(A16, 4, 4, A32, None, None) == status("FP8_ERR_DEVICE")
    assert L.fp8_swiglu_bwd(A16, A48, 4, 4, A32, A16, None) == status("FP8_ERR_DEVICE")
    assert L.fp8_swiglu_fwd(None, 0, 4, None, A16, None) == status("FP8_ERR_DEVICE")   # the amax clear


def test_scale_cast_amax_argument_checks():
    f = L.fp8_scale_cast_amax
    assert f(A16, 0, -5, A32, 0, A48, A16, None) == status("FP8_ERR_SIZE")
    assert f(A16, 3, 5, A32, 0, A48, A16, None) == status("FP8_ERR_DTYPE")
    assert f(A16, 0, 5, A32, 3, A48, A16, None) == status("FP8_ERR_FORMAT")
    assert f(A16, 0, 5, A32, 0, A48, None, None) == status("FP8_ERR_NULL")
    assert f(A16, 0, 5, A32, 0, A48, P(18), None) == status("FP8_ERR_ALIGN")
    assert f(None, 0, 5, A32, 0, A48, A16, None) == status("FP8_ERR_NULL")
    assert f(A16, 0, 5, None, 0, A48, A16, None) == status("FP8_ERR_NULL")
    assert f(A16, 0, 5, A32, 0, None, A16, None) == status("FP8_ERR_NULL")
    assert f(MIS, 0, 5, A32, 0, A48, A16, None) == status("FP8_ERR_ALIGN")
    assert f(A16, 1, 5, A32, 0, MIS, A16, None) == status("FP8_ERR_ALIGN")


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_scale_cast_amax_without_a_device_reports_no_device():
    # even n == 0 clears the amax output, so it needs the device
    assert L.fp8_scale_cast_amax(None, 0, 0, None, 0, None, A16, None) == status("FP8_ERR_DEVICE")
    assert L.fp8_scale_cast_amax(A16, 0, 5, A32, 2, A48, A16, None) == status("FP8_ERR_DEVICE")



def test_quantize_delayed_argument_checks():
    f = L.fp8_quantize_delayed
    assert f(A16, 0, -1, 0, 0, A48, A32, A32, None) == status("FP8_ERR_SIZE")
    assert f(A16, 2, 10, 0, 0, A48, A32, A32, None) == status("FP8_ERR_DTYPE")
    assert f(A16, 0, 10, 3, 0, A48, A32, A32, None) == status("FP8_ERR_FORMAT")
    assert f(A16, 0, 10, 0, 65, A48, A32, A32, None) == status("FP8_ERR_MARGIN")
    assert f(None, 0, 10, 0, 0, A48, A32, A32, None) == status("FP8_ERR_NULL")
    assert f(A16, 0, 10, 0, 0, None, A32, A32, None) == status("FP8_ERR_NULL")
    assert f(A16, 0, 10, 0, 0, A48, None, A32, None) == status("FP8_ERR_NULL")
    assert f(A16, 0, 10, 0, 0, A48, A32, None, None) == status("FP8_ERR_NULL")
    assert f(MIS, 0, 10, 0, 0, A48, A32, A32, None) == status("FP8_ERR_ALIGN")
    assert f(A16, 0, 10, 0, 0, MIS, A32, A32, None) == status("FP8_ERR_ALIGN")
    assert f(A16, 0, 10, 0, 0, A48, P(18), A32, None) == status("FP8_ERR_ALIGN")
    assert f(A16, 0, 10, 0, 0, A48, A32, P(18), None) == status("FP8_ERR_ALIGN")


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_quantize_delayed_without_a_device_reports_no_device():
    # n == 0 still writes the bias and clears the amax
    assert L.fp8_quantize_delayed(None, 0, 0, 0, 0, None, A16, A32, None) == status("FP8_ERR_DEVICE")
    assert L.fp8_quantize_delayed(A16, 0, 5, 0, 0, A48, A16, A32, None) == status("FP8_ERR_DEVICE")


def test_quantize_argument_checks():
    f = L.fp8_quantize
    assert f(A16, 0, -1, 0, 0, A48, A32, A32, None) == status("FP8_ERR_SIZE")
    assert f(A16, 2, 10, 0, 0, A48, A32, A32, None) == status("FP8_ERR_DTYPE")
    assert f(A16, 0, 10, 3, 0, A48, A32, A32, None) == status("FP8_ERR_FORMAT")
    assert f(A16, 0, 10, 0, 65, A48, A32, A32, None) == status("FP8_ERR_MARGIN")
    assert f(A16, 0, 10, 0, -65, A48, A32, A32, None) == status("FP8_ERR_MARGIN")
    assert f(None, 0, 10, 0, 0, A48, A32, A32, None) == status("FP8_ERR_NULL")
    assert f(A16, 0, 10, 0, 0, None, A32, A32, None) == status("FP8_ERR_NULL")
    assert f(A16, 0, 10, 0, 0, A48, None, A32, None) == status("FP8_ERR_NULL")
    assert f(A16, 0, 10, 0, 0, A48, A32, None, None) == status("FP8_ERR_NULL")
    # amax and bias are written even for an empty tensor, so they are needed
    assert f(None, 0, 0, 0, 0, None, None, A32, None) == status("FP8_ERR_NULL")
    assert f(MIS, 0, 10, 0, 0, A48, A32, A32, None) == status("FP8_ERR_ALIGN")
    assert f(A16, 1, 10, 0, 0, MIS, A32, A32, None) == status("FP8_ERR_ALIGN")
    assert f(A16, 0, 10, 0, 0, A48, P(18), A32, None) == status("FP8_ERR_ALIGN")
    assert f(A16, 0, 10, 0, 0, A48, A32, P(34), None) == status("FP8_ERR_ALIGN")


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_quantize_without_a_device_reports_no_device():
    assert L.fp8_quantize(A16, 0, 10, 0, 0, A48, A32, A32, None) == status("FP8_ERR_DEVICE")
    assert L.fp8_quantize(None, 1, 0, 2, 3, None, A32, A32, None) == status("FP8_ERR_DEVICE")


def test_gemm_workspace_bytes():
    f = L.fp8_scaled_gemm_workspace_bytes
    FWD, DGRAD, WGRAD = 0, 1, 2
    # 2048 x 768 output (96 tiles of 128 x 128), contraction 3072 (48 stages): 2 slices
    assert f(FWD, 2048, 768, 3072) == 2 * 2048 * 768 * 4
    assert f(DGRAD, 2048, 3072, 768) == 2 * 2048 * 768 * 4      # dX[M x K], contraction N
    assert f(WGRAD, 3072, 2304, 768) == 2 * 2304 * 768 * 4      # dW[N x K] (108 tiles), contraction M
    assert f(FWD, 2048, 768, 2304) == 0           # 36 stages: two slices would be under 24 stages
    # 128 x 8192 output (64 tiles), contraction 8192: 4 slices (one workgroup
    # per CU; five, the most of 24 stages, would leave 64 CUs with two)
    assert f(FWD, 128, 8192, 8192) == 4 * 128 * 8192 * 4
    # 192 x 10240 (160 tiles), contraction 8192: 3 slices, two workgroups on
    # most CUs (one per CU would leave it unsplit); 65 x 28672 (224 tiles): 2;
    # 128 x 28672 (224 tiles): none (adding two slices of 14.7 MB costs what
    # sharing the CUs saves)
    assert f(FWD, 192, 10240, 8192) == 3 * 192 * 10240 * 4
    assert f(FWD, 65, 28672, 8192) == 2 * 65 * 28672 * 4
    assert f(FWD, 128, 28672, 8192) == 0
    # one tile, contraction of 240 stages: 10 slices of 24 stages
    assert f(FWD, 100, 100, 240 * 64) == 10 * 100 * 100 * 4
    assert f(FWD, 8192, 8192, 8192) == 0          # fills the chip
    assert f(FWD, 2048, 2304, 768) == 0           # 288 tiles
    assert f(FWD, 128, 8192, 100) == 0            # contraction not whole 64-byte stages
    assert f(FWD, 128, 128, 192) == 0             # too short to split
    assert f(FWD, 0, 128, 4096) == 0
    assert f(5, 128, 128, 4096) == status("FP8_ERR_OP")
    assert f(FWD, -1, 128, 4096) == status("FP8_ERR_SIZE")


def test_gemm_ws_argument_checks():
    f = L.fp8_scaled_gemm_ws
    split = (0, 0, A16, 0, A32, A48, 0, A32, 2048, 768, 3072, A16)      # needs 12 MiB of workspace
    need = 2 * 2048 * 768 * 4
    assert f(*split, None, need, None) == status("FP8_ERR_NULL")
    assert f(*split, MIS, need, None) == status("FP8_ERR_ALIGN")
    assert f(*split, A48, need - 1, None) == status("FP8_ERR_SIZE")
    assert f(*split, A48, -1, None) == status("FP8_ERR_SIZE")
    assert f(9, 0, A16, 0, A32, A48, 0, A32, 64, 64, 64, A16, A48, need, None) == status("FP8_ERR_OP")
    assert f(0, 0, A16, 2, A32, A48, 0, A32, 64, 64, 64, A16, A48, need, None) == status("FP8_ERR_FORMAT")
    # an empty output needs nothing
    assert f(0, 0, None, 0, None, None, 0, None, 0, 768, 3072, None, None, 0, None) == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_gemm_ws_without_a_device_reports_no_device():
    f = L.fp8_scaled_gemm_ws
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 2048, 768, 3072, A16, A48, 2 * 2048 * 768 * 4, None) \
        == status("FP8_ERR_DEVICE")
    # a product that is not split needs no workspace
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 8192, 8192, 8192, A16, None, 0, None) == status("FP8_ERR_DEVICE")


def test_gemm_noalloc_argument_checks(monkeypatch):
    """fp8_scaled_gemm_noalloc: the product checks of fp8_scaled_gemm, and a
    split that would need more than the static scratch is refused on the host
    before any device call (the default plans never do: at most 256 / tiles
    slices of an output of that many 128 x 128 tiles, 16 MiB)."""
    f = L.fp8_scaled_gemm_noalloc
    assert f(9, 0, A16, 0, A32, A48, 0, A32, 64, 64, 64, A16, None) == status("FP8_ERR_OP")
    assert f(0, 5, A16, 0, A32, A48, 0, A32, 64, 64, 64, A16, None) == status("FP8_ERR_OP")
    assert f(0, 0, A16, 2, A32, A48, 0, A32, 64, 64, 64, A16, None) == status("FP8_ERR_FORMAT")
    assert f(0, 0, A16, 0, None, A48, 0, A32, 64, 64, 64, A16, None) == status("FP8_ERR_NULL")
    assert f(0, 0, MIS, 0, A32, A48, 0, A32, 64, 64, 64, A16, None) == status("FP8_ERR_ALIGN")
    assert f(0, 0, A16, 0, A32, A48, 0, A32, -1, 64, 64, A16, None) == status("FP8_ERR_SIZE")
    assert f(0, 0, None, 0, None, None, 0, None, 0, 768, 3072, None, None) == 0
    # the largest plan of one workgroup per CU fits exactly: 64 slices of a 4-tile output
    ws = L.fp8_scaled_gemm_workspace_bytes
    assert ws(0, 256, 256, 64 * 24 * 64) == 64 * 256 * 256 * 4 == fl.NOALLOC_SCRATCH_BYTES
    # a caller's workspace may be planned for two workgroups per CU past the
    # scratch: 192 x 10240 in 3 slices, 23.6 MB (the no-allocation product
    # then runs it unsplit)
    assert ws(0, 192, 10240, 8192) == 3 * 192 * 10240 * 4 > fl.NOALLOC_SCRATCH_BYTES
    # more planned slots: a 4-tile output split 256 ways needs 64 MiB
    monkeypatch.setenv("FP8LIN_SPLIT_SLOTS", "4096")
    assert ws(0, 256, 256, 256 * 24 * 64) == 256 * 256 * 256 * 4
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 256, 256, 256 * 24 * 64, A16, None) == status("FP8_ERR_SIZE")


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_gemm_noalloc_without_a_device_reports_no_device():
    """Past the size checks, the call needs a device: products split, unsplit,
    and split by a plan smaller than a caller's workspace would get (its own
    fits the static scratch, so no size error)."""
    f = L.fp8_scaled_gemm_noalloc
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 2048, 768, 3072, A16, None) == status("FP8_ERR_DEVICE")
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 8192, 8192, 8192, A16, None) == status("FP8_ERR_DEVICE")
    assert L.fp8_scaled_gemm_workspace_bytes(0, 192, 10240, 8192) > fl.NOALLOC_SCRATCH_BYTES
    assert f(0, 0, A16, 0, A32, A48, 0, A32, 192, 10240, 8192, A16, None) == status("FP8_ERR_DEVICE")


def _qdesc(x=A16, n=10, dtype=0, fmt=0, margin=0, y=A48, amax=A32, bias=A32):
    return fl.QuantDesc(x.value if isinstance(x, P) else x, n, dtype, fmt, margin, 0,
                        y.value if isinstance(y, P) else y, amax.value if isinstance(amax, P) else amax,
                        bias.value if isinstance(bias, P) else bias)


def test_quantize_multi_argument_checks():
    f = L.fp8_quantize_multi
    ok = _qdesc()
    arr = lambda *ds: (fl.QuantDesc * len(ds))(*ds)
    assert f(None, -1, None) == status("FP8_ERR_SIZE")
    assert f(None, 0, None) == 0
    assert f(None, 2, None) == status("FP8_ERR_NULL")
    # the first bad descriptor's fp8_quantize status, nothing launched
    assert f(arr(ok, _qdesc(n=-1)), 2, None) == status("FP8_ERR_SIZE")
    assert f(arr(ok, _qdesc(dtype=4)), 2, None) == status("FP8_ERR_DTYPE")
    assert f(arr(ok, _qdesc(fmt=3)), 2, None) == status("FP8_ERR_FORMAT")
    assert f(arr(ok, _qdesc(margin=65)), 2, None) == status("FP8_ERR_MARGIN")
    assert f(arr(ok, _qdesc(x=None)), 2, None) == status("FP8_ERR_NULL")
    assert f(arr(ok, _qdesc(amax=None)), 2, None) == status("FP8_ERR_NULL")
    assert f(arr(ok, _qdesc(x=MIS)), 2, None) == status("FP8_ERR_ALIGN")
    assert f(arr(ok, _qdesc(bias=P(34))), 2, None) == status("FP8_ERR_ALIGN")
    assert f(arr(_qdesc(fmt=9), _qdesc(n=-3)), 2, None) == status("FP8_ERR_FORMAT")
    # an empty tensor needs no input or output pointers (its amax and bias are written)
    assert f(arr(ok, _qdesc(x=None, y=None, n=0), _qdesc(x=None, n=0, amax=None)), 3, None) == status("FP8_ERR_NULL")


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_quantize_multi_without_a_device_reports_no_device():
    arr = (fl.QuantDesc * 2)(_qdesc(), _qdesc(n=0, x=None, y=None))
    assert L.fp8_quantize_multi(arr, 2, None) == status("FP8_ERR_DEVICE")


def _gdesc(op=0, fa=0, fb=0, a=A16, ba=A32, b=A48, bb=A32, M=64, N=64, K=64, out=A16):
    v = lambda p: p.value if isinstance(p, P) else p
    return fl.GemmDesc(op, fa, fb, 0, v(a), v(ba), v(b), v(bb), M, N, K, v(out))


def test_gemm_group_argument_checks():
    f, wsb = L.fp8_scaled_gemm_group, L.fp8_scaled_gemm_group_workspace_bytes
    arr = lambda *ds: (fl.GemmDesc * len(ds))(*ds)
    ok = _gdesc()
    assert wsb(0, None, 0) == 0 and f(0, None, 0, None, 0, None) == 0
    assert wsb(0, None, -1) == status("FP8_ERR_SIZE") and wsb(0, arr(ok), 257) == status("FP8_ERR_SIZE")
    assert wsb(0, None, 1) == status("FP8_ERR_NULL")
    assert wsb(2, arr(ok), 1) == status("FP8_ERR_OP")
    assert wsb(0, arr(ok, _gdesc(op=3)), 2) == status("FP8_ERR_OP")
    assert wsb(0, arr(ok, _gdesc(fa=2)), 2) == status("FP8_ERR_FORMAT")
    assert wsb(0, arr(ok, _gdesc(out=None)), 2) == status("FP8_ERR_NULL")
    assert wsb(0, arr(ok, _gdesc(ba=None)), 2) == status("FP8_ERR_NULL")
    assert wsb(0, arr(ok, _gdesc(a=MIS)), 2) == status("FP8_ERR_ALIGN")
    assert wsb(0, arr(ok, _gdesc(bb=P(34))), 2) == status("FP8_ERR_ALIGN")
    assert wsb(0, arr(ok, _gdesc(M=-1)), 2) == status("FP8_ERR_SIZE")
    # the same status from the call itself, before anything runs
    assert f(0, arr(ok, _gdesc(fa=2)), 2, None, 0, None) == status("FP8_ERR_FORMAT")
    # empty products need nothing
    assert f(0, arr(_gdesc(M=0, a=None, out=None), _gdesc(op=2, N=0, a=None, b=None, out=None)), 2,
             None, 0, None) == 0


def test_gemm_group_workspace_plan():
    """A launch splits a product along the contraction only into slices of at
    least its average work per workgroup slot (512 of them; tile-stages /
    512, at least 8 stages), the blocks balancing by longest-first order
    otherwise.  The GPT-111M layer's nine products at 2048 tokens (38016
    tile-stages, 75 per slot) are one training-step launch without a split;
    each pass alone (12672 tile-stages, 25 per slot) splits its 32- to
    48-stage products in two.  A product of 1024 tiles or more, or whose
    contraction is not a whole number of 64-byte stages, runs alone."""
    wsb = L.fp8_scaled_gemm_group_workspace_bytes
    T = 2048
    lin = [("qkv", 768, 2304), ("up", 768, 3072), ("down", 3072, 768)]
    fwd = [_gdesc(0, M=T, N=n, K=k) for _, k, n in lin]
    dgrad = [_gdesc(1, 1, 0, M=T, N=n, K=k) for _, k, n in lin]
    wgrad = [_gdesc(2, 1, 0, M=T, N=n, K=k) for _, k, n in lin]
    arr = lambda ds: (fl.GemmDesc * len(ds))(*ds)
    r = lambda b: (b + 255) // 256 * 256
    assert wsb(0, arr(fwd + dgrad + wgrad), 9) == 0
    assert wsb(0, arr(fwd), 3) == r(2 * T * 768 * 4)                       # down (48 stages)
    assert wsb(0, arr(dgrad), 3) == 2 * r(2 * T * 768 * 4)                 # qkv (36), up (48)
    assert wsb(0, arr(wgrad), 3) == r(2 * 2304 * 768 * 4) + r(2 * 3072 * 768 * 4) + r(2 * 768 * 3072 * 4)
    # one 128 x 128 tile of 40 stages: 5 slices of 8; with an 8-stage one beside it, the same
    one = _gdesc(0, M=128, N=128, K=64 * 40)
    assert wsb(0, arr([one]), 1) == r(5 * 128 * 128 * 4)
    assert wsb(0, arr([_gdesc(0, M=128, N=128, K=64 * 8), one]), 2) == r(5 * 128 * 128 * 4)
    # run alone, no workspace: 8192 x 8192 (4096 tiles), K = 100
    assert wsb(0, arr([_gdesc(0, M=8192, N=8192, K=64 * 40)]), 1) == 0
    assert wsb(0, arr([_gdesc(0, M=128, N=128, K=100)]), 1) == 0
    # 128 tokens through a 70B QKV projection (80 tiles of 128 stages): 7 slices
    assert wsb(0, arr([_gdesc(0, M=128, N=10240, K=8192)]), 1) == r(7 * 128 * 10240 * 4)
    # 64 tokens or fewer through a weight of 16 MiB or more: alone in the row
    # kernel, no workspace (under 16 MiB: grouped and split)
    assert wsb(0, arr([_gdesc(0, M=64, N=10240, K=8192)]), 1) == 0
    assert wsb(0, arr([_gdesc(0, M=64, N=1024, K=8192)]), 1) > 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on a real device")
def test_gemm_group_without_a_device_reports_no_device():
    arr = (fl.GemmDesc * 1)(_gdesc())
    assert L.fp8_scaled_gemm_group(0, arr, 1, None, 0, None) == status("FP8_ERR_DEVICE")
