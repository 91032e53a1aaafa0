"""Pins of the oracle's FP8 GEMMs (CPU only).

Definition: "Training and inference of large language models using 8-bit
floating point", review page, "Proposed method", bullet 3 (the product of the
scaled FP8 operands is unscaled after the matmul) and bullet 5 (the method is
used in training, so forward, data-gradient and weight-gradient products):
    fwd   Y  = 2^-(bx+bw)  * X8 . W8^T     X8: MxK, W8: NxK
    dgrad dX = 2^-(bdy+bw) * dY8 . W8      dY8: MxN, W8: NxK
    wgrad dW = 2^-(bdy+bx) * dY8^T . X8    dY8: MxN, X8: MxK

Independent references: exact rational arithmetic (fractions.Fraction) on tiny
shapes, torch's float64 matmul on the torch-decoded operands (one layout
mistake -- a transposed operand, a swapped index -- changes these), the
identity matrix, K = 1 and all-zero special cases.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

E4M3, E5M2 = 0, 1
TORCH_FMT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
PAIRS = [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)]


def torch_decode(codes, fmt):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(TORCH_FMT[fmt]).to(torch.float64)


def finite_codes(rng, shape, fmt):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    if fmt == E4M3:
        bad = (c & 0x7F) == 0x7F
    else:
        bad = (c & 0x7F) >= 0x7C
    c[bad] = c[bad] & 0xF0 | 0x01 if fmt == E4M3 else c[bad] & 0x80 | 0x33
    return c


def frac_value(code, fmt):
    code = int(code)
    s = -1 if code & 0x80 else 1
    if fmt == E4M3:
        E, M = (code >> 3) & 15, code & 7
        mag = Fraction(M, 2 ** 9) if E == 0 else Fraction(8 + M) * Fraction(2) ** (E - 10)
    else:
        E, M = (code >> 2) & 31, code & 3
        mag = Fraction(M, 2 ** 16) if E == 0 else Fraction(4 + M) * Fraction(2) ** (E - 17)
    return s * mag


def assert_fp64_sum(got, terms, scale, exact_required):
    """got must be the fp64 sum of the exact products `terms` times `scale`:
    exact when every partial sum is representable (E4M3 x E4M3: multiples of
    2^-18 below 2^53), else within the recursive-summation bound
    (n-1) * 2^-53 * sum|t| (each product is exact in fp64)."""
    exact = sum(terms) * scale
    mag = sum(abs(t) for t in terms) * scale
    err = abs(Fraction(got) - exact)
    if exact_required:
        assert err == 0, (got, exact)
    else:
        assert err <= max(len(terms) - 1, 0) * Fraction(1, 2 ** 53) * mag, (got, exact)


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_tiny_shapes_exact_rationals(orc, fa, fb):
    rng = np.random.default_rng(fa * 10 + fb)
    for trial in range(12):
        M, N, K = (int(v) for v in rng.integers(1, 7, 3))
        ba, bb = (int(v) for v in rng.integers(-20, 30, 2))
        scale = Fraction(2) ** (-(ba + bb))
        # fwd: X8 (fa) MxK, W8 (fb) NxK
        x8, w8 = finite_codes(rng, (M, K), fa), finite_codes(rng, (N, K), fb)
        y, bd = orc.gemm_fwd(x8, fa, ba, w8, fb, bb)
        for i in range(M):
            for j in range(N):
                terms = [frac_value(x8[i, k], fa) * frac_value(w8[j, k], fb) for k in range(K)]
                assert_fp64_sum(y[i, j], terms, scale, fa == fb == E4M3)
                assert_fp64_sum(bd[i, j], [abs(t) for t in terms], scale, fa == fb == E4M3)
        # dgrad: dY8 (fa) MxN, W8 (fb) NxK
        dy8 = finite_codes(rng, (M, N), fa)
        dx, bd = orc.gemm_dgrad(dy8, fa, ba, w8, fb, bb)
        for i in range(M):
            for k in range(K):
                terms = [frac_value(dy8[i, j], fa) * frac_value(w8[j, k], fb) for j in range(N)]
                assert_fp64_sum(dx[i, k], terms, scale, fa == fb == E4M3)
                assert_fp64_sum(bd[i, k], [abs(t) for t in terms], scale, fa == fb == E4M3)
        # wgrad: dY8 (fa) MxN, X8 (fb) MxK
        xb = finite_codes(rng, (M, K), fb)
        dw, bd = orc.gemm_wgrad(dy8, fa, ba, xb, fb, bb)
        for j in range(N):
            for k in range(K):
                terms = [frac_value(dy8[i, j], fa) * frac_value(xb[i, k], fb) for i in range(M)]
                assert_fp64_sum(dw[j, k], terms, scale, fa == fb == E4M3)
                assert_fp64_sum(bd[j, k], [abs(t) for t in terms], scale, fa == fb == E4M3)


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_layouts_match_torch_float64_matmul(orc, fa, fb):
    rng = np.random.default_rng(100 + fa * 10 + fb)
    M, N, K = 37, 53, 71
    ba, bb = 6, 12
    s = 2.0 ** -(ba + bb)
    x8, w8 = finite_codes(rng, (M, K), fa), finite_codes(rng, (N, K), fb)
    y, bd = orc.gemm_fwd(x8, fa, ba, w8, fb, bb)
    X, W = torch_decode(x8, fa), torch_decode(w8, fb)
    ref = (X @ W.T).numpy() * s
    assert np.allclose(y, ref, rtol=1e-15, atol=0)
    assert np.allclose(bd, (X.abs() @ W.abs().T).numpy() * s, rtol=1e-15, atol=0)
    # a transposed operand would not match (guards the test itself)
    assert not np.allclose(y[:, :M], (X @ X.T).numpy()[:, :M] * s)

    dy8 = finite_codes(rng, (M, N), fa)
    dx, bd = orc.gemm_dgrad(dy8, fa, ba, w8, fb, bb)
    DY = torch_decode(dy8, fa)
    assert np.allclose(dx, (DY @ W).numpy() * s, rtol=1e-15, atol=0)
    assert np.allclose(bd, (DY.abs() @ W.abs()).numpy() * s, rtol=1e-15, atol=0)

    xb = finite_codes(rng, (M, K), fb)
    dw, bd = orc.gemm_wgrad(dy8, fa, ba, xb, fb, bb)
    XB = torch_decode(xb, fb)
    assert np.allclose(dw, (DY.T @ XB).numpy() * s, rtol=1e-15, atol=0)
    assert np.allclose(bd, (DY.abs().T @ XB.abs()).numpy() * s, rtol=1e-15, atol=0)


def test_identity_weight_returns_unscaled_input(orc):
    rng = np.random.default_rng(4)
    M, K = 19, 32
    x8 = finite_codes(rng, (M, K), E4M3)
    eye = np.where(np.eye(K, dtype=bool), 0x38, 0x00).astype(np.uint8)   # E4M3 1.0 = 0x38
    y, _ = orc.gemm_fwd(x8, E4M3, 5, eye, E4M3, 0)
    assert np.array_equal(y, orc.decode_fp8(x8, E4M3) * 2.0 ** -5)
    # dgrad against the identity returns dY itself; wgrad with X = I returns dY^T
    dy8 = finite_codes(rng, (K, K), E5M2)
    dx, _ = orc.gemm_dgrad(dy8, E5M2, 3, eye, E4M3, 0)
    assert np.array_equal(dx, orc.decode_fp8(dy8, E5M2) * 2.0 ** -3)
    dw, _ = orc.gemm_wgrad(dy8, E5M2, 3, eye, E4M3, 0)
    assert np.array_equal(dw, orc.decode_fp8(dy8, E5M2).T * 2.0 ** -3)


def test_k1_is_a_single_exact_product_and_zero_is_exact(orc):
    rng = np.random.default_rng(6)
    x8, w8 = finite_codes(rng, (9, 1), E4M3), finite_codes(rng, (7, 1), E4M3)
    y, _ = orc.gemm_fwd(x8, E4M3, -3, w8, E4M3, 2)
    ref = np.outer(orc.decode_fp8(x8[:, 0], E4M3), orc.decode_fp8(w8[:, 0], E4M3)) * 2.0
    assert np.array_equal(y, ref)
    z = np.zeros((5, 64), dtype=np.uint8)
    y, bd = orc.gemm_fwd(z, E4M3, 0, finite_codes(rng, (6, 64), E4M3), E4M3, 0)
    assert np.all(y == 0) and np.all(bd == 0)
    # K = 0: empty sums are zero
    y, bd = orc.gemm_fwd(np.zeros((3, 0), np.uint8), E4M3, 0, np.zeros((4, 0), np.uint8), E4M3, 0)
    assert y.shape == (3, 4) and np.all(y == 0)


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_sampled_outputs_equal_full_outputs(orc, which):
    rng = np.random.default_rng(8)
    M, N, K = 45, 38, 29
    a8 = finite_codes(rng, (M, K if which == "fwd" else N), E5M2)
    if which == "fwd":
        b8 = finite_codes(rng, (N, K), E4M3)
        full, fbd = orc.gemm_fwd(a8, E5M2, 7, b8, E4M3, -2)
        at = orc.gemm_fwd_at
    elif which == "dgrad":
        b8 = finite_codes(rng, (N, K), E4M3)
        full, fbd = orc.gemm_dgrad(a8, E5M2, 7, b8, E4M3, -2)
        at = orc.gemm_dgrad_at
    else:
        b8 = finite_codes(rng, (M, K), E4M3)
        full, fbd = orc.gemm_wgrad(a8, E5M2, 7, b8, E4M3, -2)
        at = orc.gemm_wgrad_at
    rows = rng.integers(0, full.shape[0], 500)
    cols = rng.integers(0, full.shape[1], 500)
    out, bd = at(a8, E5M2, 7, b8, E4M3, -2, rows, cols)
    assert np.array_equal(out, full[rows, cols])
    assert np.array_equal(bd, fbd[rows, cols])


# (X8 row in E5M2, W8 row in E4M3) -> the expected output and its bound under
# the IEEE reading of special codes: a NaN term, inf * 0 or inf - inf gives
# NaN; otherwise an infinite term gives that infinity (E5M2 0x7C = +inf,
# 0xFC = -inf, 0x3C = 1; E4M3 0x38 = 1, 0xB8 = -1, 0x7F = NaN)
SPECIAL_CASES = [
    ([0x7C, 0x3C], [0x38, 0x38], np.inf, np.inf),
    ([0xFC, 0x3C], [0x38, 0x38], -np.inf, np.inf),
    ([0x7C, 0x3C], [0xB8, 0x38], -np.inf, np.inf),
    ([0x7C, 0xFC], [0x38, 0x38], np.nan, np.inf),      # inf - inf; the magnitudes still add
    ([0x7C, 0x3C], [0x00, 0x38], np.nan, np.nan),      # inf * 0
    ([0x7F, 0x3C], [0x38, 0x38], np.nan, np.nan),      # an E5M2 NaN code
    ([0x3C, 0x3C], [0x7F, 0x38], np.nan, np.nan),      # an E4M3 NaN code
    ([0x3C, 0x3C], [0xFF, 0x00], np.nan, np.nan),      # -NaN
]


@pytest.mark.parametrize("x,w,want,want_bound", SPECIAL_CASES)
def test_special_codes_follow_ieee_arithmetic(orc, x, w, want, want_bound):
    x8 = np.array([x], dtype=np.uint8)
    w8 = np.array([w], dtype=np.uint8)
    for bias in (0, 5, -7):
        y, bound = orc.gemm_fwd(x8, E5M2, bias, w8, E4M3, 0)
        for got, exp in ((y[0, 0], want), (bound[0, 0], want_bound)):
            if np.isnan(exp):
                assert np.isnan(got)
            else:
                assert got == exp
        # the same terms through the two gradient layouts
        dx, _ = orc.gemm_dgrad(x8, E5M2, bias, w8.T.copy(), E4M3, 0)
        dw, _ = orc.gemm_wgrad(x8.T.copy(), E5M2, bias, w8.T.copy(), E4M3, 0)
        for got in (dx[0, 0], dw[0, 0]):
            assert (np.isnan(got) and np.isnan(want)) or got == want


# ------------------------------------------------------------ accumulation
# oracle.gemm_accumulate: old + product.  Pins: a zero buffer gives the
# product itself; accumulating the product over the second half of the
# contraction onto the first half's equals the whole contraction's product
# (linearity of the sum; a dropped, negated or transposed buffer fails it);
# all-zero operands leave the buffer as it was.

CONTRACTION_AXES = {0: (1, 1), 1: (1, 0), 2: (0, 0)}   # op -> (axis of a, axis of b)


def _halves(x, axis, h):
    return (np.ascontiguousarray(np.take(x, np.arange(h), axis=axis)),
            np.ascontiguousarray(np.take(x, np.arange(h, x.shape[axis]), axis=axis)))


@pytest.mark.parametrize("op", [0, 1, 2])
def test_accumulate_is_linear_in_the_contraction(orc, op):
    rng = np.random.default_rng(50 + op)
    shapes = {0: ((12, 40), (9, 40)), 1: ((12, 40), (40, 9)), 2: ((40, 12), (40, 9))}[op]
    fa, fb = (E4M3, E4M3) if op == 0 else (E5M2, E4M3)
    a = finite_codes(rng, shapes[0], fa)
    b = finite_codes(rng, shapes[1], fb)
    ba, bb = 3, -2
    gemm = (orc.gemm_fwd, orc.gemm_dgrad, orc.gemm_wgrad)[op]
    full, bound = gemm(a, fa, ba, b, fb, bb)
    ax_a, ax_b = CONTRACTION_AXES[op]
    a1, a2 = _halves(a, ax_a, 17)
    b1, b2 = _halves(b, ax_b, 17)
    first, _ = gemm(a1, fa, ba, b1, fb, bb)
    # the first half's product rounded to the fp32 buffer it would sit in
    old = first.astype(np.float32)
    acc, bd = orc.gemm_accumulate(op, old, a2, fa, ba, b2, fb, bb)
    second, _ = gemm(a2, fa, ba, b2, fb, bb)
    assert np.array_equal(acc, old.astype(np.float64) + second)
    # against the whole contraction: only the buffer's fp32 rounding differs
    assert np.all(np.abs(acc - full) <= 2.0 ** -24 * np.abs(first) + 1e-12 * bound)
    assert not np.allclose(acc, full - 2 * second)             # a negated product would land here
    zero = np.zeros_like(old)
    acc0, bd0 = orc.gemm_accumulate(op, zero, a2, fa, ba, b2, fb, bb)
    assert np.array_equal(acc0, second) and np.array_equal(bd0, bd)
    # all-zero operands: the buffer comes back unchanged
    za, zb = np.zeros_like(a2), np.zeros_like(b2)
    same, _ = orc.gemm_accumulate(op, old, za, fa, ba, zb, fb, bb)
    assert np.array_equal(same, old.astype(np.float64))
    with pytest.raises(ValueError):                            # a transposed buffer
        orc.gemm_accumulate(op, np.ascontiguousarray(old.T), a2, fa, ba, b2, fb, bb)
