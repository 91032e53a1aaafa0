"""How gfx950's MFMA instructions sum their products, measured one
instruction at a time (tests/hip/mfma_probe.hip), and what that means for the
products' tolerance |err| <= 1e-5 * 2^-(ba+bb) * sum |a||b| ("Training and
inference of large language models using 8-bit floating point", review page,
"Proposed method", bullet 3: FP8 operands, matmul, unscale).

  * Window: output (0, 0) = b + s - b with b = 2^16 and s = b * 2^-g, the
    three terms in different contraction positions.  The largest g for which
    every placement returns s exactly is the instruction's window: 13 for
    every FP8 instruction (v_mfma_scale_f32_{32x32x64,16x16x128}_f8f6f4,
    v_mfma_f32_32x32x16_{fp8,bf8}_{fp8,bf8}), 23 for the 16-bit ones
    (v_mfma_f32_32x32x16_{f16,bf16}) on FP8 values widened exactly -- as
    wide as the fp32 accumulator's own 24-bit significand.
  * One instruction on random FP8-valued operands: the FP8 instructions
    miss 1e-5 * sum |a||b| by themselves; the 16-bit ones are at fp32 level.
  * The native FP8 path (fp8_scaled_gemm, FP8_GEMM_NATIVE_FP8) over every
    product of the five workloads: always within the bound the window implies
    (tests/mfma_bound.py); within 1e-5 * sum |a||b| on four of them, but not
    on the Llama-2-7B MLP with its outlier-heavy activations (the exact
    path meets 1e-5 on all five, test_gpu_gemm.py::test_workload_products).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_gemm, i32_dev, need_gpu, say, u8_dev
from mfma_bound import native_bound, native_bound_at

pytestmark = pytest.mark.gpu
E4M3, E5M2 = 0, 1
LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libmfma_probe.so")

# kind: (probe id, output rows, output cols, contraction per instruction, 16-bit operands)
KINDS = {
    "f8f6f4_32x32x64": (0, 32, 32, 64, False),
    "f8f6f4_16x16x128": (1, 16, 16, 128, False),
    "fp8_32x32x16": (2, 32, 32, 16, False),
    "f16_32x32x16": (3, 32, 32, 16, True),
    "bf16_32x32x16": (4, 32, 32, 16, True),
}
WINDOW = {"f8f6f4_32x32x64": 13, "f8f6f4_16x16x128": 13, "fp8_32x32x16": 13,
          "f16_32x32x16": 23, "bf16_32x32x16": 23}


@pytest.fixture(scope="module")
def probe():
    need_gpu()
    assert os.path.exists(LIB), f"{LIB} is not built: python tests/hip/build_probe.py"
    lib = ctypes.CDLL(LIB)
    lib.probe_mfma.restype = ctypes.c_int
    lib.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p]
    return lib


def codes_of(values, fmt):
    dt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(dt)
    assert torch.equal(t.to(torch.float64), torch.tensor(np.asarray(values, dtype=np.float64))), "not exact"
    return t.view(torch.uint8).numpy()


def words_of(values, kind):
    v = np.asarray(values, dtype=np.float32)
    if kind == "f16_32x32x16":
        w = v.astype(np.float16)
        assert np.array_equal(w.astype(np.float32), v)
        return w.view(np.uint16)
    t = torch.tensor(v).to(torch.bfloat16)
    assert np.array_equal(t.float().numpy(), v)
    return t.view(torch.int16).numpy().view(np.uint16)


def images(kind, A, B):
    """Per-lane register images (64 x 32 bytes) of A [rows x k] and B [k x cols]."""
    kid, rows, cols, kk, wide = KINDS[kind]
    a = np.zeros((64, 32), dtype=np.uint8)
    b = np.zeros((64, 32), dtype=np.uint8)
    per = 32 if kid in (0, 1) else 8          # contraction elements per lane
    for l in range(64):
        r, h = l % rows, l // rows
        ka = A[r, per * h:per * (h + 1)]
        kb = B[per * h:per * (h + 1), l % cols]
        if wide:
            a[l, :16] = np.ascontiguousarray(ka, dtype=np.uint16).view(np.uint8)
            b[l, :16] = np.ascontiguousarray(kb, dtype=np.uint16).view(np.uint8)
        else:
            a[l, :per] = ka
            b[l, :per] = kb
    return a, b


def run(probe, kind, fa, fb, A, B):
    kid, rows, cols, kk, wide = KINDS[kind]
    a, b = images(kind, A, B)
    out = np.zeros((64, 16), dtype=np.float32)
    rc = probe.probe_mfma(kid, fa, fb, a.ctypes.data, b.ctypes.data, out.ctypes.data)
    assert rc == 0, rc
    C = np.zeros((rows, cols), dtype=np.float32)
    for l in range(64):
        if rows == 32:
            for r in range(16):
                C[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] = out[l, r]
        else:
            for r in range(4):
                C[4 * (l // 16) + r, l % 16] = out[l, r]
    return C


def operand(kind, values, fmt):
    return words_of(values, kind) if KINDS[kind][4] else codes_of(values, fmt)


FORMATS = [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)]


@pytest.mark.parametrize("kind", list(KINDS))
def test_register_layout(probe, kind):
    """The probe's register images are the instruction's operand layout: small
    integers (every sum exact in any window) multiply as A @ B."""
    kid, rows, cols, kk, wide = KINDS[kind]
    rng = np.random.default_rng(kid)
    for fa, fb in (FORMATS[:1] if wide else FORMATS):
        Av = rng.integers(-4, 5, (rows, kk)).astype(np.float64)
        Bv = rng.integers(-4, 5, (kk, cols)).astype(np.float64)
        say("mfma layout", kind, fa, fb)
        C = run(probe, kind, fa, fb, operand(kind, Av, fa), operand(kind, Bv, fb))
        assert np.array_equal(C.astype(np.float64), Av @ Bv), kind


def _power_split(e, lo_a, lo_b):
    """(ea, eb) with ea + eb = e, each at least its format's smallest power."""
    ea = max(lo_a, e - 8)
    return ea, e - ea


@pytest.mark.parametrize("kind", list(KINDS))
def test_summation_window(probe, kind):
    kid, rows, cols, kk, wide = KINDS[kind]
    placements = [(0, 1, 2), (kk - 1, kk // 2, 0), (3, kk - 2, kk // 2 + 1), (kk // 2 - 1, 5, kk - 3)]
    lo = {E4M3: -9, E5M2: -16}
    windows = []
    for fa, fb in (FORMATS[:2] if wide else FORMATS):
        first_lost = None
        for g in range(1, 35):
            ea, eb = _power_split(16 - g, lo[fa], lo[fb])
            exact = True
            for (k0, k1, k2) in placements:
                Av = np.zeros((rows, kk))
                Bv = np.zeros((kk, cols))
                Av[0, k0], Bv[k0, 0] = 2.0 ** 8, 2.0 ** 8          # b = 2^16
                Av[0, k1], Bv[k1, 0] = 2.0 ** ea, 2.0 ** eb        # s = 2^(16 - g)
                Av[0, k2], Bv[k2, 0] = -(2.0 ** 8), 2.0 ** 8       # -b
                C = run(probe, kind, fa, fb, operand(kind, Av, fa), operand(kind, Bv, fb))
                exact &= C[0, 0] == 2.0 ** (16 - g)
            if not exact:
                first_lost = g
                break
        window = (first_lost - 1) if first_lost else 34
        print(f"{kind} fmts {fa},{fb}: b + s - b exact for g <= {window}")
        windows.append(window)
    assert min(windows) == max(windows) == WINDOW[kind], (kind, windows)


@pytest.mark.parametrize("kind", list(KINDS))
def test_single_instruction_error_on_workload_like_values(probe, kind):
    """One instruction on FP8 values of N(0, 1) draws scaled into E4M3's
    range (the activations' distribution): the FP8 instructions' error exceeds
    1e-5 * sum |a||b| at some output, the 16-bit ones stay at fp32 level."""
    kid, rows, cols, kk, wide = KINDS[kind]
    rng = np.random.default_rng(40 + kid)
    worst = 0.0
    for trial in range(24):
        Av = torch.tensor(rng.standard_normal((rows, kk)) * 64, dtype=torch.float32).to(
            torch.float8_e4m3fn).to(torch.float64).numpy()
        Bv = torch.tensor(rng.standard_normal((kk, cols)) * 64, dtype=torch.float32).to(
            torch.float8_e4m3fn).to(torch.float64).numpy()
        C = run(probe, kind, E4M3, E4M3, operand(kind, Av, E4M3), operand(kind, Bv, E4M3))
        exact = Av @ Bv
        mag = np.abs(Av) @ np.abs(Bv)
        worst = max(worst, float(np.max(np.abs(C - exact) / mag)))
        if not wide:    # within the window's bound, instruction by instruction
            check_gemm(C, exact, native_bound(Av, Bv, 0), f"{kind} trial {trial}", rel=1.0)
    print(f"{kind}: worst err / sum|ab| over one instruction = {worst:.3e}")
    if wide:
        assert worst <= 1e-6
    else:
        assert worst > 1e-5


def _workload_operands(w, name, cache):
    if name not in cache:
        t = w.tensor(name)
        words = synth.bf16_words(synth.workload_tensor(w, name))
        _, b, codes = oracle.quantize(words, t.fmt, t.margin)
        cache[name] = (codes, b, t.fmt)
    return cache[name]


@pytest.mark.parametrize("wl", [1, 2, 3, 4, 5])
def test_native_path_on_the_workloads(wl):
    """Every product of each workload in native FP8 arithmetic, in the launch
    configuration the benchmark uses (split products included), against the
    oracle: every output of workload 1; for the others 4096 random outputs
    and the first 32 x 32 block of each product.  Each output is within the window's bound; the
    worst err / sum |a||b| per product is recorded against 1e-5."""
    fl = need_gpu()
    w = synth.WORKLOADS[wl]
    rng = np.random.default_rng(500 + wl)
    cache = {}
    worst = {}
    op_of = {"fwd": fl.OP_FWD, "dgrad": fl.OP_DGRAD, "wgrad": fl.OP_WGRAD}
    at_of = {"fwd": oracle.gemm_fwd_at, "dgrad": oracle.gemm_dgrad_at, "wgrad": oracle.gemm_wgrad_at}
    for l in w.linears:
        for which in l.passes:
            an, bn = {"fwd": (l.x, l.w), "dgrad": (l.dy, l.w), "wgrad": (l.dy, l.x)}[which]
            a8, ba, fa = _workload_operands(w, an, cache)
            b8, bb, fb = _workload_operands(w, bn, cache)
            rows_out, cols_out = {"fwd": (l.M, l.N), "dgrad": (l.M, l.K), "wgrad": (l.N, l.K)}[which]
            nbytes = fl.gemm_workspace_bytes(op_of[which], l.M, l.N, l.K)
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
            say("native workload", wl, l.name, which, l.M, l.N, l.K)
            got = fl.scaled_gemm(op_of[which], u8_dev(a8), fa, i32_dev(ba), u8_dev(b8), fb, i32_dev(bb),
                                 math=fl.MATH_NATIVE_FP8, workspace=ws).cpu().numpy()
            if wl == 1:
                rows, cols = (v.ravel() for v in np.meshgrid(np.arange(rows_out), np.arange(cols_out),
                                                             indexing="ij"))
            else:   # 4096 random outputs and the first 32 x 32 block
                b32 = np.arange(32)
                fr, fc = (v.ravel() for v in np.meshgrid(b32, b32, indexing="ij"))
                rows = np.concatenate([rng.integers(0, rows_out, 4096), fr])
                cols = np.concatenate([rng.integers(0, cols_out, 4096), fc])
            ref, mag = at_of[which](a8, fa, ba, b8, fb, bb, rows, cols)
            splits = nbytes // (rows_out * cols_out * 4) if nbytes else 0
            bound = native_bound_at(which, a8, fa, b8, fb, rows, cols, -(ba + bb), extra=splits)
            g = got[rows, cols].astype(np.float64)
            check_gemm(g, ref, bound, f"native wl{wl} {l.name} {which}", rel=1.0)
            worst[f"{l.name}:{which}"] = float(np.max(np.abs(g - ref) / np.where(mag > 0, mag, 1.0)))
            del got
    print(f"workload {wl} native FP8 worst err / sum|ab| per product:",
          {k: f"{v:.3e}" for k, v in worst.items()}, "(bar 1e-5)")
    # measured: the native arithmetic meets the bar on the normal-valued
    # workloads and misses it on the Llama-2-7B MLP, whose Student-t
    # activations with outliers spread each instruction's products over more
    # binades than its window keeps (worst 1.6e-4 on the up product) -- why the
    # library's default products are exact
    if wl == 3:
        assert max(worst.values()) > 1e-5, worst
    else:
        assert max(worst.values()) <= 1e-5, worst
