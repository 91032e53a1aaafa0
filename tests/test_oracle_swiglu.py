"""Pins of the oracle's SwiGLU step (CPU only).

The activation between the two products of the chained FP8 MLP is Llama 2's
SwiGLU (the pages train Llama 2 models, "Training and inference of large
language models using 8-bit floating point", review page, "Main findings",
without spelling the activation out): a = silu(g) * u, silu(g) = g * sigmoid(g),
with h = [g | u] the up-projection's output (gate columns first).

Independent references, none sharing code with the oracle:
  * torch.nn.functional.silu in float64, and torch.autograd of silu(g) * u;
  * central finite differences of the oracle's own forward;
  * closed forms: silu(0) = 0, silu'(0) = 1/2, silu(g) -> g and silu'(g) -> 1
    as g -> inf, silu(g) -> 0 as g -> -inf, and the zero of silu' near
    g = -1.2785 (root of 1 + g * (1 - sigmoid(g)), found here by bisection).
"""
import math

import numpy as np
import torch


def split(h):
    f = h.shape[1] // 2
    return h[:, :f].astype(np.float64), h[:, f:].astype(np.float64)


def draw(rows, f, seed, scale=3.0):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((rows, 2 * f)) * scale).astype(np.float32)
    da = rng.standard_normal((rows, f)).astype(np.float32)
    return h, da


def test_forward_matches_torch_silu(orc):
    h, _ = draw(37, 129, 1)
    g, u = split(h)
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    got = orc.swiglu_fwd(h)
    assert got.shape == (37, 129)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-300)


def test_backward_matches_torch_autograd(orc):
    h, da = draw(23, 77, 2)
    g, u = split(h)
    tg = torch.from_numpy(g).requires_grad_()
    tu = torch.from_numpy(u).requires_grad_()
    (torch.nn.functional.silu(tg) * tu).backward(torch.from_numpy(da.astype(np.float64)))
    got = orc.swiglu_bwd(h, da)
    f = g.shape[1]
    np.testing.assert_allclose(got[:, :f], tg.grad.numpy(), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(got[:, f:], tu.grad.numpy(), rtol=1e-12, atol=1e-300)


def test_backward_matches_finite_differences(orc):
    """d/dg and d/du of sum(da * a) by central differences of the forward."""
    h, da = draw(4, 50, 3, scale=2.0)
    f = 50
    dh = orc.swiglu_bwd(h, da)
    eps = 2.0 ** -12
    for col in range(2 * f):
        hp, hm = h.astype(np.float64).copy(), h.astype(np.float64).copy()
        hp[:, col] += eps
        hm[:, col] -= eps
        # h +- eps stays exact in float32 (|h| < 2^11, eps = 2^-12 ... within 24 bits)
        assert np.array_equal(hp.astype(np.float32).astype(np.float64), hp)
        ap = orc.swiglu_fwd(hp.astype(np.float32))
        am = orc.swiglu_fwd(hm.astype(np.float32))
        num = ((ap - am) * da.astype(np.float64)).sum(axis=1) / (2 * eps)
        np.testing.assert_allclose(dh[:, col], num, rtol=1e-5, atol=1e-7)


def test_closed_forms(orc):
    g = np.array([0.0, 40.0, 80.0, -40.0, -80.0, -1000.0, 1000.0], dtype=np.float32)
    u = np.array([3.0, 2.0, -1.5, 2.0, 1.0, 5.0, 0.5], dtype=np.float32)
    h = np.concatenate([g, u])[None, :]
    da = np.array([[2.0, 1.0, 1.0, 1.0, 1.0, 1.0, 4.0]], dtype=np.float32)
    a = orc.swiglu_fwd(h)[0]
    dh = orc.swiglu_bwd(h, da)[0]
    n = g.size
    assert a[0] == 0.0                                    # silu(0) = 0
    assert dh[0] == 2.0 * 3.0 * 0.5 and dh[n] == 0.0      # silu'(0) = 1/2
    assert a[1] == 40.0 * 2.0 and a[2] == 80.0 * -1.5     # sigmoid(40) = 1 - 4e-18 -> 1
    # silu'(40) = 1 + 40 e^-40 (1 + O(e^-40)) = 1 + 1.7e-16
    assert abs(dh[1] - 2.0 * (1 + 40.0 * math.exp(-40.0))) <= 4.5e-16 and dh[n + 1] == 40.0
    assert a[6] == 500.0 and dh[6] == 0.5 * 4.0 and dh[n + 6] == 4000.0
    # g = -40, -80: silu(g) = g e^g / (1 + e^g), silu'(g) = e^g (1 + g) (1 + O(e^g))
    for i, gv in ((3, -40.0), (4, -80.0)):
        e = math.exp(gv)
        assert abs(a[i] - gv * e / (1 + e) * float(u[i])) <= 1e-15 * abs(a[i])
        assert abs(dh[i] - float(da[0, i]) * float(u[i]) * e * (1 + gv)) <= 1e-14 * abs(dh[i])
    assert a[5] == 0.0 and np.signbit(a[5])               # -1000 * e^-1000 -> -0


def test_derivative_zero(orc):
    """silu' vanishes where 1 + g * (1 - sigmoid(g)) = 0 (bisection here)."""
    lo, hi = -2.0, -1.0
    F = lambda x: 1.0 + x * (1.0 - 1.0 / (1.0 + math.exp(-x)))
    for _ in range(200):
        mid = (lo + hi) / 2
        if F(mid) > 0:
            hi = mid
        else:
            lo = mid
    g0 = np.float32(lo)
    h = np.array([[g0, 1.0]], dtype=np.float32)
    dh = orc.swiglu_bwd(h, np.array([[1.0]], dtype=np.float32))
    assert abs(dh[0, 0]) < 1e-6
    assert abs(lo + 1.2784645) < 1e-6


def test_non_finite_inputs_follow_ieee(orc):
    g = np.array([np.inf, -np.inf, np.nan, 1.0], dtype=np.float32)
    u = np.array([2.0, 2.0, 2.0, np.inf], dtype=np.float32)
    a = orc.swiglu_fwd(np.concatenate([g, u])[None, :])[0]
    assert a[0] == np.inf
    assert np.isnan(a[1])            # -inf * sigmoid(-inf) = -inf * 0
    assert np.isnan(a[2])
    assert a[3] == np.inf
