"""Pins of the oracle's per-tensor amax and compute_bias (CPU only).

Definitions: "Training and inference of large language models using 8-bit
floating point", review page, "Proposed method", bullet 1 (per-tensor maximum
absolute value for weights, activations and gradients) and bullet 2
(compute_bias: log2 of format max over tensor amplitude, configurable margin).
The floor, the subtracted margin and the 0/inf/NaN conventions are this
library's readings.

Independent references: Python's float arithmetic for max|x| on small inputs,
torch.amax, a brute-force search "largest integer b with amax * 2^b <= fmt_max"
(math.ldexp, exact in double), and hand-worked values in
tests/golden/bias_closed_form.txt.
"""
import math
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
E4M3, E5M2, E3M4 = 0, 1, 2
ALL_FMTS = [E4M3, E5M2, E3M4]
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0, E3M4: 30.0}   # E3M4: the reading of the oracle's header
FMT_NAME = {"E4M3": E4M3, "E5M2": E5M2, "E3M4": E3M4}


def f32_of_bits(b):
    return float(np.array([b], dtype=np.uint32).view(np.float32)[0])


def bits_of_f32(x):
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def bf16_words_of(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def python_amax(values):
    """max |x| with the library's NaN / inf conventions, in plain Python."""
    best = 0.0
    for v in values:
        if math.isnan(v):
            return float("nan")
        best = max(best, abs(v))
    return best


def bias_bruteforce(a, fmt_max, margin):
    """Largest integer b with a * 2^b <= fmt_max, minus margin (a > 0 finite)."""
    b = 0
    while math.ldexp(a, b) > fmt_max:
        b -= 1
    while math.ldexp(a, b + 1) <= fmt_max:
        b += 1
    return b - margin


# ---------------------------------------------------------------- amax
def test_amax_small_inputs_bruteforce(orc):
    rng = np.random.default_rng(1)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32)
        w = x.view(np.uint32)
        assert orc.amax(x) == np.float32(python_amax([float(v) for v in x]))
        xb = bf16_words_of(x)
        vals = torch.from_numpy(xb.astype(np.int16)).view(torch.bfloat16).float().tolist()
        assert orc.amax(xb) == np.float32(python_amax(vals))
        # permutation invariance and membership
        p = rng.permutation(n)
        assert orc.amax_bits(w[p]) == orc.amax_bits(w)
        assert orc.amax(x) in set(np.abs(x).tolist())


def test_amax_matches_torch_on_large_finite(orc):
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_t(3, 1_000_003).astype(np.float32))
    xb = x.to(torch.bfloat16)
    words = xb.view(torch.int16).numpy().view(np.uint16)
    assert orc.amax(words) == torch.amax(xb.abs()).float().item()
    assert orc.amax(x.numpy()) == torch.amax(x.abs()).item()


def test_amax_special_values(orc):
    w = lambda *v: np.array(v, dtype=np.uint16)
    assert orc.amax_bits(np.zeros(0, dtype=np.uint16)) == 0           # empty -> +0
    assert orc.amax_bits(w(0x8000, 0x8000)) == 0                      # -0 only -> +0
    assert orc.amax_bits(w(0x3F80, 0xFF80)) == 0x7F800000             # -inf -> +inf
    assert orc.amax_bits(w(0x7F80, 0x7FC1, 0xFFC5, 0x3F80)) == 0x7FC50000  # NaN: largest magnitude bits
    assert orc.amax_bits(w(0x0001)) == 0x00010000                     # bf16 subnormal widens exactly
    assert orc.amax_bits(w(0xC2F7, 0x42F6)) == 0x42F70000             # sign ignored
    f = np.array([1.0, -np.inf, np.nan], dtype=np.float32)
    assert np.isnan(orc.amax(f))
    assert orc.amax_bits(np.array([0x80000001, 0x00000000], dtype=np.uint32)) == 0x00000001


def test_amax_every_bf16_word(orc):
    words = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert orc.amax_bits(words) == 0x7FFF0000          # the NaN of largest magnitude bits
    finite = words[(words & 0x7F80) != 0x7F80]
    assert orc.amax_bits(finite) == 0x7F7F0000         # largest finite bf16


# ---------------------------------------------------------------- bias
def _golden():
    rows = []
    with open(os.path.join(HERE, "golden", "bias_closed_form.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                rows.append(line)
    return rows


def test_bias_golden_values(orc):
    rows = _golden()
    assert len(rows) >= 20
    for fmt_s, bits, margin, expected in rows:
        got = orc.compute_bias(int(bits, 16), FMT_NAME[fmt_s], int(margin))
        assert got == int(expected), (fmt_s, bits, margin, got, expected)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_bias_every_positive_finite_bf16(orc, fmt):
    words = np.arange(1, 0x7F80, dtype=np.uint32)       # +subnormals .. +max finite
    assert words.size == 32639
    bits = words << 16
    vals = bits.astype(np.uint32).view(np.float32).astype(np.float64)
    for margin in (0, 1, -2, 5):
        got = np.array([orc.compute_bias(int(b), fmt, margin) for b in bits])
        ref = np.array([bias_bruteforce(float(a), FMT_MAX[fmt], margin) for a in vals])
        bad = np.where(got != ref)[0]
        assert bad.size == 0, (margin, vals[bad[:5]], got[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_bias_fp32_thresholds_and_random(orc, fmt):
    rng = np.random.default_rng(9)
    mants = [0, 1, 0x5FFFFF, 0x600000, 0x600001, 0x6FFFFF, 0x700000, 0x700001, 0x7FFFFF, 0x400000]
    bits = [(e << 23) | m for e in range(0, 255) for m in mants if (e, m) != (0, 0)]
    bits += rng.integers(1, 0x7F800000, 30_000).tolist()
    for k in range(-150, 112):  # fmt_max * 2^k and its fp32 neighbours
        v64 = math.ldexp(FMT_MAX[fmt], k)
        if v64 < 2.0 ** -149 or v64 > 3.0e38:
            continue
        a = np.float32(v64)
        if a > 0:
            for v in (a, np.nextafter(a, np.float32(np.inf)), np.nextafter(a, np.float32(0))):
                if v > 0 and np.isfinite(v):
                    bits.append(bits_of_f32(v))
    for b in bits:
        a = f32_of_bits(b)
        assert orc.compute_bias(b, fmt, 0) == bias_bruteforce(a, FMT_MAX[fmt], 0), hex(b)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_bias_next_float_above_power_of_two_multiple_drops_by_one(orc, fmt):
    for k in range(-20, 20):
        a = np.float32(math.ldexp(FMT_MAX[fmt], -k))
        up = np.nextafter(a, np.float32(np.inf))
        assert orc.compute_bias(bits_of_f32(a), fmt, 0) == k
        assert orc.compute_bias(bits_of_f32(up), fmt, 0) == k - 1


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_bias_invariants(orc, fmt):
    words = np.arange(1, 0x7F80, dtype=np.uint32)
    bits = (words << 16).astype(np.uint32)
    vals = bits.view(np.float32).astype(np.float64)
    b0 = np.array([orc.compute_bias(int(b), fmt, 0) for b in bits])
    # monotone non-increasing in amax (words are in increasing value order)
    assert np.all(np.diff(b0) <= 0)
    # amax * 2^bias lands in (fmt_max / 2, fmt_max]
    scaled = vals * np.exp2(b0.astype(np.float64))
    assert np.all(scaled <= FMT_MAX[fmt]) and np.all(scaled > FMT_MAX[fmt] / 2)
    # the margin shifts the bias one for one
    for m in (-7, -1, 1, 4, 64):
        sample = bits[::97]
        bm = np.array([orc.compute_bias(int(b), fmt, m) for b in sample])
        assert np.array_equal(bm, b0[::97] - m)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_bias_of_zero_inf_nan_is_zero(orc, fmt):
    for bits in (0x00000000, 0x80000000, 0x7F800000, 0x7FC00000, 0x7FFFFFFF):
        for m in (-3, 0, 2):
            assert orc.compute_bias(bits, fmt, m) == 0
