"""GPU parity of amax, compute_bias and scale-then-cast against the CPU oracle.

All three must match bit for bit ("Training and inference of large language
models using 8-bit floating point", review page, "Proposed method", bullets
1-4), and so must the E3M4 cast (the third format of "Efficient post-training
quantization with FP8 formats", summary page, under the encoding the oracle's
header states).  Every call goes through the C ABI (the ctypes binding).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bf16_dev, f32_dev, i32_dev, need_gpu, say, words_of

pytestmark = pytest.mark.gpu
E4M3, E5M2, E3M4 = 0, 1, 2
ALL_FMTS = [E4M3, E5M2, E3M4]


@pytest.fixture(scope="module")
def fl():
    return need_gpu()


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_cast_every_bf16_word_for_every_bias(fl, fmt):
    words = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_dev(words)
    biases = list(range(-140, 161)) + [-200, 221]
    out = torch.empty((len(biases), 65536), dtype=torch.uint8, device="cuda")
    say("cast all bf16 words", "fmt", fmt, "biases", biases[0], "..", biases[-1])
    for r, b in enumerate(biases):
        fl.scale_cast(x, i32_dev(b), fmt, out=out[r])
    got = out.cpu().numpy()
    for r, b in enumerate(biases):
        ref = oracle.scale_cast(words, b, fmt)
        if not np.array_equal(got[r], ref):
            bad = np.where(got[r] != ref)[0][:8]
            raise AssertionError(f"fmt {fmt} bias {b}: words {words[bad]} gpu {got[r][bad]} oracle {ref[bad]}")


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_cast_fp32_words(fl, fmt):
    rng = np.random.default_rng(21)
    words = rng.integers(0, 2 ** 32, 2_000_003, dtype=np.uint64).astype(np.uint32)
    e = rng.integers(95, 150, 1_000_000).astype(np.uint32)
    words[:1_000_000] = (words[:1_000_000] & 0x807FFFFF) | (e << 23)
    words[1_000_000:1_000_100] = np.arange(100, dtype=np.uint32)       # fp32 subnormals
    x = f32_dev(words)
    for b in (-150, -40, -6, 0, 1, 9, 17, 64, 140, 220):
        say("cast fp32 words", "fmt", fmt, "bias", b, "n", words.size)
        got = fl.scale_cast(x, i32_dev(b), fmt).cpu().numpy()
        ref = oracle.scale_cast(words, b, fmt)
        assert np.array_equal(got, ref), f"bias {b}: {np.count_nonzero(got != ref)} codes differ"


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_cast_fp32_midpoints_and_neighbours(fl, fmt):
    """fp32 inputs at every midpoint between neighbouring FP8 values (and the
    one above the largest), at every FP8 value, and one fp32 ulp either side of
    each, both signs, scaled by 2^-b for biases across the range; plus the
    saturation bound fmt_max * 2^-b and its neighbours."""
    vals = oracle.decode_fp8(np.arange(128), fmt)
    vals = vals[np.isfinite(vals)]
    top = vals[-1] + (vals[-1] - vals[-2]) / 2
    pts = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2, [top]])
    fmax = {E4M3: 448.0, E5M2: 57344.0, E3M4: 30.0}[fmt]
    for b in (-127, -100, -60, -20, -9, -1, 0, 1, 7, 20, 60, 100, 126, 127, 140):
        with np.errstate(over="ignore"):
            x = np.concatenate([pts, [fmax]]) * 2.0 ** -b
            x32 = x.astype(np.float32)
        x32 = x32[np.isfinite(x32) & (x32.astype(np.float64) == x)]
        near = np.concatenate([x32, np.nextafter(x32, np.float32(np.inf)), np.nextafter(x32, np.float32(0))])
        near = near[np.isfinite(near)]
        words = np.concatenate([near, -near]).astype(np.float32).view(np.uint32)
        say("cast fp32 midpoints", "fmt", fmt, "bias", b, "n", words.size)
        got = fl.scale_cast(f32_dev(words), i32_dev(b), fmt).cpu().numpy()
        ref = oracle.scale_cast(words, b, fmt)
        if not np.array_equal(got, ref):
            bad = np.where(got != ref)[0][:6]
            raise AssertionError(f"fmt {fmt} bias {b}: words {[hex(w) for w in words[bad]]} gpu {got[bad]} oracle {ref[bad]}")


@pytest.mark.parametrize("n", [1, 7, 8, 9, 15, 16, 17, 31, 33, 255, 4097, 1_000_003])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_amax_and_cast_ragged_sizes(fl, n, dtype):
    rng = np.random.default_rng(n)
    v = (rng.standard_normal(n) * 3).astype(np.float32)
    if dtype == "bf16":
        words = synth.bf16_words(torch.from_numpy(v).to(torch.bfloat16))
        x = bf16_dev(words)
    else:
        words = v.view(np.uint32)
        x = f32_dev(words)
    say("ragged", dtype, "n", n)
    a = fl.amax(x)
    assert int(words_of(a)[0]) == oracle.amax_bits(words)
    for fmt, margin in ((E4M3, 0), (E5M2, 2), (E4M3, -1), (E3M4, 1)):
        b = fl.compute_bias(a, fmt, margin)
        assert int(b.item()) == oracle.compute_bias(oracle.amax_bits(words), fmt, margin)
        y = fl.scale_cast(x, b, fmt).cpu().numpy()
        assert np.array_equal(y, oracle.scale_cast(words, int(b.item()), fmt))


def test_amax_special_values_anywhere(fl):
    rng = np.random.default_rng(3)
    n = 100_003
    base = synth.bf16_words(torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16))
    cases = {"+inf": 0x7F80, "-inf": 0xFF80, "nan": 0x7FC0, "-nan big": 0xFFFF, "huge": 0x7F7F,
             "-huge": 0xFF7F, "subnormal only": None}
    for name, w in cases.items():
        for pos in (0, 5, n // 2, n - 9, n - 1):     # head, inside a vector, middle, tail
            words = base.copy()
            if w is None:
                words = (np.arange(n) % 0x7F + 1).astype(np.uint16)     # all bf16 subnormals
            else:
                words[pos] = w
            say("amax special", name, "pos", pos)
            got = int(words_of(fl.amax(bf16_dev(words)))[0])
            assert got == oracle.amax_bits(words), (name, pos, hex(got))
    # empty tensor -> +0 (the clear still runs)
    a = torch.full((1,), 7.0, device="cuda")
    fl.lib.fp8_amax(None, 0, 0, a.data_ptr(), None)
    torch.cuda.synchronize()
    assert a.item() == 0.0


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_bias_every_positive_bf16_amax(fl, fmt):
    words = np.arange(1, 0x7F80, dtype=np.uint32)
    step = 1 if fmt == E4M3 else 5
    bits = (words[::step] << 16).astype(np.uint32)
    amax = f32_dev(bits)
    out = torch.empty(bits.size, dtype=torch.int32, device="cuda")
    say("bias sweep", fmt, bits.size)
    for i in range(bits.size):
        fl.compute_bias(amax[i:i + 1], fmt, 0, out=out[i:i + 1])
    got = out.cpu().numpy()
    ref = np.array([oracle.compute_bias(int(b), fmt, 0) for b in bits])
    assert np.array_equal(got, ref)
    # margins and special amax values
    specials = [0, 0x80000000, 0x7F800000, 0x7FC00000, 1, 0x7F7FFFFF, 0x43E00000, 0x43E00001,
                0x41F00000, 0x41F00001, 0x41EFFFFF]
    for s in specials:
        for m in (-64, -3, 0, 1, 64):
            b = fl.compute_bias(f32_dev(np.array([s], np.uint32)), fmt, m)
            assert int(b.item()) == oracle.compute_bias(s, fmt, m), (hex(s), m)


@pytest.mark.parametrize("wl", [1, 2, 3, 4, 5])
def test_workload_tensors_bit_exact(fl, wl):
    w = synth.WORKLOADS[wl]
    for t in w.tensors:
        x = synth.workload_tensor(w, t.name)
        words = synth.bf16_words(x)
        say("workload", wl, t.name, tuple(t.shape), "fmt", t.fmt, "margin", t.margin)
        codes, bias, amax = fl.quantize(x.cuda(), t.fmt, t.margin)
        a_ref = oracle.amax_bits(words)
        b_ref = oracle.compute_bias(a_ref, t.fmt, t.margin)
        assert int(words_of(amax)[0]) == a_ref, t.name
        assert int(bias.item()) == b_ref, t.name
        got = codes.cpu().numpy().reshape(-1)
        ref = oracle.scale_cast(words.reshape(-1), b_ref, t.fmt)
        assert np.array_equal(got, ref), f"{t.name}: {np.count_nonzero(got != ref)} codes differ"
        # the cast that folds its own input's amax, with the bias just derived
        say("workload", wl, t.name, "fused cast + amax")
        am = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
        fused = fl.scale_cast(x.cuda(), bias, t.fmt, amax=am).cpu().numpy().reshape(-1)
        assert int(words_of(am)[0]) == a_ref, t.name
        assert np.array_equal(fused, ref), f"{t.name}: {np.count_nonzero(fused != ref)} fused codes differ"
        del codes, x, fused


@pytest.mark.parametrize("wl", [1, 3, 5])
def test_e3m4_quantisation_of_workload_activations(fl, wl):
    """The workload's E4M3 tensors (activations and weights) quantised to E3M4
    instead: amax, bias (fmt_max 30) and codes bit-exact, margins 0 and 1."""
    w = synth.WORKLOADS[wl]
    for t in w.tensors:
        if t.fmt != E4M3:
            continue
        x = synth.workload_tensor(w, t.name)
        words = synth.bf16_words(x)
        a_ref = oracle.amax_bits(words)
        for margin in (0, 1):
            say("E3M4 workload", wl, t.name, tuple(t.shape), "margin", margin)
            codes, bias, amax = fl.quantize(x.cuda(), E3M4, margin)
            b_ref = oracle.compute_bias(a_ref, E3M4, margin)
            assert int(words_of(amax)[0]) == a_ref, t.name
            assert int(bias.item()) == b_ref, t.name
            got = codes.cpu().numpy().reshape(-1)
            ref = oracle.scale_cast(words.reshape(-1), b_ref, E3M4)
            assert np.array_equal(got, ref), f"{t.name}: {np.count_nonzero(got != ref)} codes differ"
            del codes
        del x


def test_cast_mixes_non_finite_values_into_finite_units(fl):
    """The cast converts 16-element units on the hardware path unless a unit
    holds an inf or NaN; here every unit mixes a few of them into finite
    values (including ones that saturate), at biases on both paths."""
    rng = np.random.default_rng(5)
    n = 16 * 4096 + 7
    v = (rng.standard_normal(n) * 300).astype(np.float32)
    words = synth.bf16_words(synth.to_bf16(v)).copy()
    specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16)
    pos = rng.integers(0, n, n // 5)
    words[pos] = specials[rng.integers(0, specials.size, pos.size)]
    x = bf16_dev(words)
    for fmt in ALL_FMTS:
        for b in (-130, -4, 0, 3, 12, 126, 127):
            say("cast mixed non-finite", "fmt", fmt, "bias", b)
            got = fl.scale_cast(x, i32_dev(b), fmt).cpu().numpy()
            ref = oracle.scale_cast(words, b, fmt)
            assert np.array_equal(got, ref), f"fmt {fmt} bias {b}: {np.count_nonzero(got != ref)} codes differ"
    # the same with fp32 inputs (their own NaN payloads included)
    w32 = v.view(np.uint32).copy()
    spec32 = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x7F800001, 0x7F7FFFFF],
                      dtype=np.uint32)
    w32[pos] = spec32[rng.integers(0, spec32.size, pos.size)]
    x32 = f32_dev(w32)
    for fmt in ALL_FMTS:
        for b in (-130, -4, 0, 3, 12, 126, 127):
            say("cast mixed non-finite fp32", "fmt", fmt, "bias", b)
            got = fl.scale_cast(x32, i32_dev(b), fmt).cpu().numpy()
            ref = oracle.scale_cast(w32, b, fmt)
            assert np.array_equal(got, ref), f"fp32 fmt {fmt} bias {b}: {np.count_nonzero(got != ref)} codes differ"


def test_gradient_underflow_control(fl):
    """The 13B backward workload's gradients (~N(0,1) x 1e-6) cast to E5M2:
    with bias 0 every value lies below the smallest E5M2 subnormal's half, so
    every code is a signed zero; with the AMAX bias the codes carry the
    values (the underflow the per-tensor scale avoids)."""
    w = synth.WORKLOADS[4]
    dy = synth.workload_tensor(w, "dY_down")
    words = synth.bf16_words(dy).ravel()
    x = bf16_dev(words)
    say("underflow control dY_down", words.size)
    zero = fl.scale_cast(x, i32_dev(0), E5M2).cpu().numpy()
    assert np.all((zero & 0x7F) == 0)
    amax = fl.amax(x)
    bias = fl.compute_bias(amax, E5M2, 0)
    b = int(bias.cpu().item())
    assert b == oracle.compute_bias(oracle.amax_bits(words), E5M2, 0)
    codes = fl.scale_cast(x, bias, E5M2).cpu().numpy()
    assert np.array_equal(codes, oracle.scale_cast(words, b, E5M2))
    assert np.count_nonzero(codes & 0x7F) > 0.99 * codes.size


def test_fixed_and_delayed_scaling(fl):
    """FP8-CSCALE and delayed scaling use the same cast with a bias the
    caller chooses ("Proposed method": the fixed-scale baseline the pages
    compare AMAX against): a bias written to device memory by the caller, or
    the bias of an earlier tensor reused on a new one.  Here a tensor that has
    grown 8x since its bias was taken saturates under the stale bias exactly
    as the rounding rule says, and not under its own AMAX bias."""
    rng = np.random.default_rng(31)
    old = synth.bf16_words(synth.to_bf16((rng.standard_normal(1 << 20) * 2.0).astype(np.float32)))
    new = synth.bf16_words(synth.to_bf16((rng.standard_normal(1 << 20) * 16.0).astype(np.float32)))
    for fmt in (E4M3, E5M2):
        say("fixed / delayed scaling", "fmt", fmt)
        # fixed scale: bias chosen by the caller
        for b in (-3, 0, 5):
            got = fl.scale_cast(bf16_dev(new), i32_dev(b), fmt).cpu().numpy()
            assert np.array_equal(got, oracle.scale_cast(new, b, fmt))
        # delayed scale: the old tensor's AMAX bias, kept on the device
        stale = fl.compute_bias(fl.amax(bf16_dev(old)), fmt, 0)
        b_old = int(stale.cpu().item())
        got = fl.scale_cast(bf16_dev(new), stale, fmt).cpu().numpy()
        assert np.array_equal(got, oracle.scale_cast(new, b_old, fmt))
        top = 0x7E if fmt == E4M3 else 0x7B
        assert np.count_nonzero((got & 0x7F) == top) > 100          # saturated under the stale bias
        fresh = fl.compute_bias(fl.amax(bf16_dev(new)), fmt, 0)
        got = fl.scale_cast(bf16_dev(new), fresh, fmt).cpu().numpy()
        assert np.count_nonzero((got & 0x7F) == top) <= 2           # only the largest values reach the top code


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_cast_with_fused_amax(fl, dtype):
    """fp8_scale_cast_amax: the codes of fp8_scale_cast and max |x| of the
    input from the same pass, both bit-exact, over ragged sizes, every format,
    biases on both conversion paths, and non-finite values anywhere."""
    rng = np.random.default_rng(17)
    for n in (1, 15, 16, 17, 1023, 1024, 1025, 4096 * 3 + 5, 300_001):
        v = (rng.standard_normal(n) * 40).astype(np.float32)
        if dtype == "bf16":
            words = synth.bf16_words(synth.to_bf16(v)).copy()
            specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1], dtype=np.uint16)
            x = bf16_dev
        else:
            words = v.view(np.uint32).copy()
            specials = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001], dtype=np.uint32)
            x = f32_dev
        for with_special in (False, True):
            w = words.copy()
            if with_special:
                w[rng.integers(0, n)] = specials[rng.integers(0, specials.size)]
            xd = x(w)
            for fmt in ALL_FMTS:
                for b in (-130, 0, 5, 127):
                    say("cast+amax", dtype, n, "special", with_special, "fmt", fmt, "bias", b)
                    am = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
                    got = fl.scale_cast(xd, i32_dev(b), fmt, amax=am).cpu().numpy()
                    assert np.array_equal(got, oracle.scale_cast(w, b, fmt)), (n, fmt, b)
                    assert int(words_of(am)[0]) == oracle.amax_bits(w), (n, fmt, b)
    # n == 0: the amax output is cleared, nothing else happens
    am = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    assert fl.lib.fp8_scale_cast_amax(None, 0, 0, None, 0, None, am.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert am.item() == 0.0


def _fused_seams(dtype, n):
    """Element indices at the seams of fp8_scale_cast_amax's two launches for
    an n-element input: the first element, the main cast's last, the last
    workgroup's stretch's first and last, and the tail's last.  The main cast
    runs one bf16 unit (16 elements) per lane of 256-lane workgroups, or one
    fp32 chunk (1024 elements) per wave of 16-wave workgroups, and each of its
    workgroups leaves one word (16 / 32 bits) in the codes of the stretch: the
    fewest whole units / chunks that hold them all.  Inputs up to 8192 units /
    64 chunks go to the last workgroup alone."""
    size, small, per_block, words_per, cap = ((16, 8192, 256, 8, 32768) if dtype == "bf16"
                                              else (1024, 64, 16, 256, 8192))
    units = n // size
    if units <= small:
        first = 0
    else:
        nb0 = min(cap, -(-units // per_block))
        first = units - -(-nb0 // words_per)
    idx = {0, max(first * size - 1, 0), first * size, units * size - 1, n - 1}
    return sorted(i for i in idx if 0 <= i < n)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_cast_with_fused_amax_at_its_seams(fl, dtype):
    """fp8_scale_cast_amax casts all but a last stretch of its input in one
    launch, each workgroup leaving its largest magnitude as a word in the code
    bytes of that stretch, then one workgroup reduces the words and casts the
    stretch over them.  Sizes on both sides of the one-workgroup limit, the
    largest magnitude or a NaN planted at each seam: codes and amax bit-exact."""
    rng = np.random.default_rng(29)
    sizes = (131072, 131072 + 3, 8193 * 16 + 3, 5_000_003) if dtype == "bf16" else \
        (65536 + 1023, 65 * 1024 + 7, 3_000_017)
    for n in sizes:
        v = (rng.standard_normal(n) * 3).astype(np.float32)
        if dtype == "bf16":
            base = synth.bf16_words(synth.to_bf16(v)).copy()
            big, nan, dev = np.uint16(0xC700), np.uint16(0x7FC0), bf16_dev   # -32768, NaN
        else:
            base = v.view(np.uint32).copy()
            big, nan, dev = np.uint32(0xC7000000), np.uint32(0x7FC00000), f32_dev
        for i in _fused_seams(dtype, n):
            for plant, val in (("largest", big), ("NaN", nan)):
                w = base.copy()
                w[i] = val
                say("cast+amax seams", dtype, n, plant, "at", i)
                am = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
                got = fl.scale_cast(dev(w), i32_dev(-8), E4M3, amax=am).cpu().numpy()
                assert int(words_of(am)[0]) == oracle.amax_bits(w), (n, plant, i)
                assert np.array_equal(got, oracle.scale_cast(w, -8, E4M3)), (n, plant, i)


def test_cast_with_fused_amax_random_sizes(fl):
    """fp8_scale_cast_amax and fp8_quantize_delayed over 40 seeded sizes from
    1 to 6M elements (both input types, every format, biases on both
    conversion paths, the largest magnitude planted at a random position):
    codes, amax and bias bit-exact against the oracle."""
    rng = np.random.default_rng(41)
    sizes = sorted(set(int(v) for v in np.exp(rng.uniform(0, np.log(6e6), 40))))
    for k, n in enumerate(sizes):
        dtype = ("bf16", "fp32")[k % 2]
        fmt, b = ALL_FMTS[k % 3], (-3, 4, 150)[(k // 3) % 3]
        v = (rng.standard_normal(n) * 5).astype(np.float32)
        v[rng.integers(0, n)] = -200.0
        if dtype == "bf16":
            words = synth.bf16_words(synth.to_bf16(v)).copy()
            x = bf16_dev(words)
        else:
            words = v.view(np.uint32).copy()
            x = f32_dev(words)
        say("cast+amax random size", dtype, n, "fmt", fmt, "bias", b)
        a_ref = oracle.amax_bits(words)
        am = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
        got = fl.scale_cast(x, i32_dev(b), fmt, amax=am).cpu().numpy()
        assert int(words_of(am)[0]) == a_ref, (n, dtype)
        assert np.array_equal(got, oracle.scale_cast(words, b, fmt)), (n, dtype, fmt, b)
        prev = torch.from_numpy(np.array([0x3F800000 + k], dtype=np.uint32).view(np.float32)).cuda()
        codes, bias = fl.quantize_delayed(x, fmt, prev, 1)
        b_ref = oracle.compute_bias(0x3F800000 + k, fmt, 1)
        assert int(bias.item()) == b_ref and int(words_of(prev)[0]) == a_ref, (n, dtype)
        assert np.array_equal(codes.cpu().numpy(), oracle.scale_cast(words, b_ref, fmt)), (n, dtype, fmt)


def test_delayed_scaling_with_the_fused_cast(fl):
    """Delayed scaling: step t casts with the bias computed from the amax the
    step t-1 cast returned (bias 0 at t = 0), and returns its own amax; every
    step's codes and amax equal the oracle's on that schedule."""
    rng = np.random.default_rng(23)
    scales = [1.0, 3.0, 0.25, 40.0, 40.0, 1e-3]
    bias = i32_dev(0)
    prev_bits = None
    for t, sc in enumerate(scales):
        v = (rng.standard_normal(65536 + 7) * sc).astype(np.float32)
        words = synth.bf16_words(synth.to_bf16(v)).copy()
        say("delayed scaling step", t)
        am = torch.empty(1, dtype=torch.float32, device="cuda")
        codes = fl.scale_cast(bf16_dev(words), bias, E4M3, amax=am).cpu().numpy()
        b_ref = 0 if prev_bits is None else oracle.compute_bias(prev_bits, E4M3, 0)
        assert int(bias.item()) == b_ref, t
        assert np.array_equal(codes, oracle.scale_cast(words, b_ref, E4M3)), t
        prev_bits = oracle.amax_bits(words)
        assert int(words_of(am)[0]) == prev_bits, t
        bias = fl.compute_bias(am, E4M3, 0)



@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_delayed(fl, dtype):
    """fp8_quantize_delayed: the bias from the amax word the previous step left
    (zero, normal, subnormal, inf and NaN amaxes at three margins), the codes
    at that bias, and this input's amax written over the word; every result
    bit-exact against the oracle, on sizes on both sides of the one-workgroup
    limit, at the two launches' seams, every format; n == 0 too."""
    rng = np.random.default_rng(31)
    prev_words = [0x0, 0x3F800000, 0x43E00000, 0x00000100, 0x7F800000, 0x7FC00000, 0x38000000]
    sizes = (17, 131072, 8193 * 16 + 3, 1_000_003) if dtype == "bf16" else (17, 65536 + 1023, 65 * 1024 + 7, 1_000_003)
    for n in sizes:
        v = (rng.standard_normal(n) * 9).astype(np.float32)
        if dtype == "bf16":
            words = synth.bf16_words(synth.to_bf16(v)).copy()
            x = bf16_dev(words)
        else:
            words = v.view(np.uint32).copy()
            x = f32_dev(words)
        a_ref = oracle.amax_bits(words)
        for k, pw in enumerate(prev_words):
            fmt, margin = ALL_FMTS[k % 3], (-2, 0, 3)[k % 3]
            say("quantize_delayed", dtype, n, "prev amax", hex(pw), "fmt", fmt, "margin", margin)
            am = torch.from_numpy(np.array([pw], dtype=np.uint32).view(np.float32)).cuda()
            codes, bias = fl.quantize_delayed(x, fmt, am, margin)
            b_ref = oracle.compute_bias(pw, fmt, margin)
            assert int(bias.item()) == b_ref, (n, hex(pw), fmt, margin)
            assert np.array_equal(codes.cpu().numpy(), oracle.scale_cast(words, b_ref, fmt)), (n, hex(pw), fmt)
            assert int(words_of(am)[0]) == a_ref, (n, hex(pw), fmt)
    # n == 0: the bias from the previous amax, and the amax of nothing
    am = torch.full((1,), 3.0, dtype=torch.float32, device="cuda")
    bias = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    assert fl.lib.fp8_quantize_delayed(None, 0, 0, E5M2, 1, None, am.data_ptr(), bias.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert am.item() == 0.0 and int(bias.item()) == oracle.compute_bias(0x40400000, E5M2, 1)


def test_delayed_scaling_in_one_call(fl):
    """A six-step delayed-scaling schedule through fp8_quantize_delayed alone:
    step t's bias from step t-1's amax (the word starts at 0: bias 0), the
    same codes, biases and amaxes as the oracle's schedule."""
    rng = np.random.default_rng(37)
    am = torch.zeros(1, dtype=torch.float32, device="cuda")
    prev_bits = 0
    for t, sc in enumerate([1.0, 3.0, 0.25, 40.0, 40.0, 1e-3]):
        v = (rng.standard_normal(300_001) * sc).astype(np.float32)
        words = synth.bf16_words(synth.to_bf16(v)).copy()
        say("delayed scaling in one call, step", t)
        codes, bias = fl.quantize_delayed(bf16_dev(words), E5M2, am, 0)
        b_ref = oracle.compute_bias(prev_bits, E5M2, 0)
        assert int(bias.item()) == b_ref, t
        assert np.array_equal(codes.cpu().numpy(), oracle.scale_cast(words, b_ref, E5M2)), t
        prev_bits = oracle.amax_bits(words)
        assert int(words_of(am)[0]) == prev_bits, t


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_degenerate_tensors(fl, dtype):
    """Tensors the method meets at its edges: all +0, all -0, mixed zeros,
    all NaN, all inf, one NaN among zeros, a constant, a single element, only
    subnormal inputs, the largest finite value.  amax (separate and folded in
    the cast), bias at three margins and codes, every format, all bit-exact."""
    n = 4099
    if dtype == "bf16":
        mk = lambda v: np.full(n, v, dtype=np.uint16)
        pz, nz, nan, inf, one, sub, big = 0x0000, 0x8000, 0x7FC0, 0x7F80, 0x3F80, 0x0001, 0x7F7F
        dev = bf16_dev
    else:
        mk = lambda v: np.full(n, v, dtype=np.uint32)
        pz, nz, nan, inf, one, sub, big = 0x0, 0x80000000, 0x7FC00000, 0x7F800000, 0x3F800000, 0x1, 0x7F7FFFFF
        dev = f32_dev
    cases = {"+0": mk(pz), "-0": mk(nz), "constant 1": mk(one), "all NaN": mk(nan), "all inf": mk(inf),
             "subnormal": mk(sub), "largest finite": mk(big)}
    mixed = mk(pz)
    mixed[::2] = nz
    cases["mixed zeros"] = mixed
    lone = mk(pz)
    lone[n // 3] = nan
    cases["one NaN"] = lone
    cases["single"] = mk(one)[:1].copy()
    for name, words in cases.items():
        x = dev(words)
        a_ref = oracle.amax_bits(words)
        assert int(words_of(fl.amax(x))[0]) == a_ref, name
        for fmt in ALL_FMTS:
            for margin in (-3, 0, 2):
                say("degenerate", dtype, name, "fmt", fmt, "margin", margin)
                codes, bias, amax = fl.quantize(x, fmt, margin)
                b_ref = oracle.compute_bias(a_ref, fmt, margin)
                assert int(bias.item()) == b_ref, (name, fmt, margin)
                ref = oracle.scale_cast(words, b_ref, fmt)
                assert np.array_equal(codes.cpu().numpy(), ref), (name, fmt, margin)
                am = torch.empty(1, dtype=torch.float32, device="cuda")
                fused = fl.scale_cast(x, bias, fmt, amax=am).cpu().numpy()
                assert np.array_equal(fused, ref) and int(words_of(am)[0]) == a_ref, (name, fmt, margin)


def _quantize_inputs(dtype, n, scale, special, seed):
    """Words of a seeded normal tensor times `scale`, with an optional planted
    NaN, inf or largest-magnitude element."""
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal(n) * scale).astype(np.float32)
    if dtype == "bf16":
        words = (torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)).copy()
        nan, inf = 0xFFC1, 0x7F80
    else:
        words = v.view(np.uint32).copy()
        nan, inf = 0x7FC00123, 0xFF800000
    if n and special == "nan":
        words[n // 2] = nan
    elif n and special == "inf":
        words[n - 1] = inf
    return words


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_in_one_call(fl, dtype, monkeypatch):
    """fp8_quantize against the oracle and against amax -> compute_bias ->
    scale_cast, bit for bit, on both of its paths (one workgroup; clear, amax
    and a cast deriving the bias itself), each forced over every size:
    ragged sizes on both sides of the 256 KiB threshold, all three
    formats, margins, biases outside the hardware conversion's range (tiny
    and huge scales) and planted NaN / inf."""
    dev = bf16_dev if dtype == "bf16" else f32_dev
    sizes = [0, 1, 7, 15, 16, 17, 1023, 4099, 16389, 65536, 65537, 131072, 131073, 1_000_003]
    for si, n in enumerate(sizes):
        for scale, special in ((1.0, None), (1e-37, None), (3e4, "inf"), (0.02, "nan")):
            words = _quantize_inputs(dtype, n, scale, special, 100 + si)
            x = dev(words)
            for fmt, margin in ((E4M3, 0), (E5M2, 1), (E3M4, -2), (E4M3, 64)):
                a_ref, b_ref, c_ref = oracle.quantize(words, fmt, margin)
                cc, cb, ca = fl.quantize_chain(x, fmt, margin)
                for path, small in (("one workgroup", "2000000000"), ("three launches", "-1"),
                                    ("default choice", None)):
                    if small is None:
                        monkeypatch.delenv("FP8LIN_QUANT_SMALL", raising=False)
                    else:
                        monkeypatch.setenv("FP8LIN_QUANT_SMALL", small)
                    say("quantize", dtype, "n", n, "scale", scale, special, "fmt", fmt, "margin", margin, path)
                    codes, bias, amax = fl.quantize(x, fmt, margin)
                    what = (dtype, n, scale, special, fmt, margin, path)
                    assert int(words_of(amax)[0]) == a_ref, what
                    assert int(bias.item()) == b_ref, what
                    got = codes.cpu().numpy()
                    assert np.array_equal(got, c_ref), what
                    assert np.array_equal(got, cc.cpu().numpy()), what
                    assert int(words_of(ca)[0]) == a_ref and int(cb.item()) == b_ref, what


def test_quantize_multi(fl):
    """fp8_quantize_multi: 41 tensors in one call (two launch groups of up to
    32), mixed sizes (empty, ragged tails, above and below one block's
    reach, up to 1M elements), bf16 and fp32, all three formats, margins,
    tiny and huge scales, planted NaN / inf: every amax, bias and code
    bit-identical to the oracle and to fp8_quantize of that tensor alone."""
    sizes = [0, 1, 7, 15, 16, 17, 255, 1023, 4099, 16389, 65536, 131073, 300001, 1_000_003]
    scales = [(1.0, None), (1e-37, None), (3e4, "inf"), (0.02, "nan")]
    fmts = [(E4M3, 0), (E5M2, 1), (E3M4, -2), (E4M3, 64), (E5M2, -3)]
    cases = []
    for i in range(41):
        dtype = "bf16" if i % 3 else "fp32"
        n = sizes[(i * 5) % len(sizes)]
        scale, special = scales[i % len(scales)]
        fmt, margin = fmts[i % len(fmts)]
        words = _quantize_inputs(dtype, n, scale, special, 900 + i)
        x = (bf16_dev if dtype == "bf16" else f32_dev)(words)
        cases.append((dtype, n, scale, special, fmt, margin, words, x))
    say("quantize_multi", len(cases), "tensors")
    got = fl.quantize_multi([c[7] for c in cases], [c[4] for c in cases], [c[5] for c in cases])
    torch.cuda.synchronize()
    for (dtype, n, scale, special, fmt, margin, words, x), (codes, bias, amax) in zip(cases, got):
        what = (dtype, n, scale, special, fmt, margin)
        a_ref, b_ref, c_ref = oracle.quantize(words, fmt, margin)
        assert int(words_of(amax)[0]) == a_ref, what
        assert int(bias.item()) == b_ref, what
        assert np.array_equal(codes.cpu().numpy(), c_ref), what
        one = fl.quantize(x, fmt, margin)
        assert torch.equal(one[0], codes) and torch.equal(one[1], bias), what
        assert torch.equal(one[2].view(torch.int32), amax.view(torch.int32)), what
    # into preallocated outputs, a second time over the same buffers
    outs = [(torch.full((c[1],), 0xAB, dtype=torch.uint8, device="cuda"),
             torch.full((1,), 77, dtype=torch.int32, device="cuda"),
             torch.full((1,), 5.0, dtype=torch.float32, device="cuda")) for c in cases]
    for _ in range(2):
        fl.quantize_multi([c[7] for c in cases], [c[4] for c in cases], [c[5] for c in cases], outs=outs)
    torch.cuda.synchronize()
    for (codes, bias, amax), (c2, b2, a2) in zip(got, outs):
        assert torch.equal(codes, c2) and torch.equal(bias, b2)
        assert torch.equal(amax.view(torch.int32), a2.view(torch.int32))


def test_quantize_multi_of_a_workload_step(fl):
    """The nine tensors quantised in the GPT-111M layer's step (X, W, dY of
    three linears) in one call, against the oracle."""
    w = synth.WORKLOADS[2]
    names = [t.name for t in w.tensors if t.timed]
    xs = [synth.workload_tensor(w, n).cuda() for n in names]
    say("quantize_multi workload 2", names)
    got = fl.quantize_multi(xs, [w.tensor(n).fmt for n in names], [w.tensor(n).margin for n in names])
    for n, x, (codes, bias, amax) in zip(names, xs, got):
        a_ref, b_ref, c_ref = oracle.quantize(synth.bf16_words(synth.workload_tensor(w, n)),
                                              w.tensor(n).fmt, w.tensor(n).margin)
        assert int(words_of(amax)[0]) == a_ref and int(bias.item()) == b_ref, n
        assert np.array_equal(codes.cpu().numpy().reshape(-1), np.asarray(c_ref).reshape(-1)), n
