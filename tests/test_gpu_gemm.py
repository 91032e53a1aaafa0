"""GPU parity of the three FP8 products against the CPU oracle.

Forward Y = X8 W8^T, data gradient dX = dY8 W8, weight gradient dW = dY8^T X8,
each unscaled by 2^-(bias_a + bias_b) ("Training and inference of large
language models using 8-bit floating point", review page, "Proposed method",
bullets 3 and 5).  The bar, elementwise:
    |gpu - oracle| <= 1e-5 * 2^-(ba+bb) * sum_k |a_k| |b_k|
so an all-zero row or column must be exactly 0.  The FP8 operands are made by
the oracle (or drawn as codes) and uploaded: nothing the GPU computed feeds
an expected value.
"""
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_gemm, i32_dev, need_gpu, say, u8_dev
from mfma_bound import native_bound, native_bound_at, operand_values

pytestmark = pytest.mark.gpu
E4M3, E5M2 = 0, 1
PAIRS = [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)]


@pytest.fixture(scope="module")
def fl():
    return need_gpu()


# Kernel configurations: the automatic choice, then each pipelined tile with
# each MFMA the exact arithmetic can run on (fp16 and bf16).
CONFIGS = [("auto", "auto"), ("128", "f16"), ("256", "f16"), ("128", "bf16"), ("256", "bf16")]


@pytest.fixture(params=CONFIGS, ids=[f"tile{t}-{m}" for t, m in CONFIGS])
def tile(request, monkeypatch):
    t, m = request.param
    for var, val in (("FP8LIN_GEMM_TILE", t), ("FP8LIN_EXACT_MFMA", m)):
        if val != "auto":
            monkeypatch.setenv(var, val)
        else:
            monkeypatch.delenv(var, raising=False)
    return f"{t}/{m}"


def finite_codes(rng, shape, fmt):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    bad = (c & 0x7F) == 0x7F if fmt == E4M3 else (c & 0x7F) >= 0x7C
    c[bad] &= 0xF0
    return c


def run(fl, which, a8, fa, ba, b8, fb, bb):
    """GPU product through the C ABI; returns a float32 numpy array."""
    A, B = u8_dev(a8), u8_dev(b8)
    BA, BB = i32_dev(ba), i32_dev(bb)
    fn = {"fwd": fl.scaled_gemm_fwd, "dgrad": fl.scaled_gemm_dgrad, "wgrad": fl.scaled_gemm_wgrad}[which]
    return fn(A, fa, BA, B, fb, BB).cpu().numpy()


def reference(which, a8, fa, ba, b8, fb, bb):
    fn = {"fwd": oracle.gemm_fwd, "dgrad": oracle.gemm_dgrad, "wgrad": oracle.gemm_wgrad}[which]
    return fn(a8, fa, ba, b8, fb, bb)


def operands(rng, which, M, N, K, fa, fb):
    """(a8, b8) in the layouts of the product: fwd X8[MxK], W8[NxK];
    dgrad dY8[MxN], W8[NxK]; wgrad dY8[MxN], X8[MxK]."""
    if which == "fwd":
        return finite_codes(rng, (M, K), fa), finite_codes(rng, (N, K), fb)
    if which == "dgrad":
        return finite_codes(rng, (M, N), fa), finite_codes(rng, (N, K), fb)
    return finite_codes(rng, (M, N), fa), finite_codes(rng, (M, K), fb)


SHAPES = [(300, 520, 392), (1, 17, 1), (64, 64, 0), (257, 129, 1000), (128, 256, 256),
          (33, 700, 130), (512, 512, 128), (260, 300, 17)]


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_small_and_ragged_shapes(fl, tile, which, fa, fb):
    rng = np.random.default_rng(zlib.crc32(f"ragged {which} {fa} {fb}".encode()))
    for (M, N, K) in SHAPES:
        a8, b8 = operands(rng, which, M, N, K, fa, fb)
        ba, bb = (int(v) for v in rng.integers(-12, 20, 2))
        say("gemm", which, "tile", tile, "fmts", fa, fb, "MNK", M, N, K)
        got = run(fl, which, a8, fa, ba, b8, fb, bb)
        ref, bound = reference(which, a8, fa, ba, b8, fb, bb)
        assert got.shape == ref.shape
        check_gemm(got, ref, bound, f"{which} {M}x{N}x{K} fmts {fa},{fb} tile {tile}")


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_identity_operand_is_exact_including_subnormals(fl, tile, which):
    """With the other operand the identity (code 0x38 = 1.0), every output is a
    single product: exact, so FP8 subnormal inputs must not be flushed."""
    rng = np.random.default_rng(17)
    n = 160
    eye = np.where(np.eye(n, dtype=bool), 0x38, 0x00).astype(np.uint8)
    codes = finite_codes(rng, (n, n), E5M2)
    codes[:, :40] = rng.integers(0, 4, (n, 40)).astype(np.uint8) | (rng.integers(0, 2, (n, 40)).astype(np.uint8) << 7)
    vals = oracle.decode_fp8(codes, E5M2)
    say("identity", which, "tile", tile)
    if which == "fwd":
        got = run(fl, which, codes, E5M2, 3, eye, E4M3, 0)
        want = vals * 2.0 ** -3
    elif which == "dgrad":
        got = run(fl, which, codes, E5M2, 3, eye, E4M3, 0)
        want = vals * 2.0 ** -3
    else:
        got = run(fl, which, codes, E5M2, 3, eye, E4M3, 0)
        want = vals.T * 2.0 ** -3
    assert np.array_equal(got.astype(np.float64), want)


# Forward products of one or two rows whose contraction is a multiple of 16
# but not of 256 run in the vector kernel: every W row streamed in 1 KB runs,
# exact fp32 products summed per run, per row and over the wave in a fixed
# order.  Rows 1 and 2, a single run (K = 16), ragged tails of a run
# (K = 1040, 8208, 32752), column counts that leave waves idle (N = 1, 17),
# the largest contraction it takes (M * K <= 64 KiB: 65520) and one past it
# (the tiled kernels then), K = 0 (the row kernel).
GEMV_SHAPES = [(1, 1000, 16), (2, 17, 1040), (1, 4103, 8208), (2, 1, 2064), (1, 256, 65520),
               (2, 96, 32752), (1, 64, 65552), (2, 40, 0)]


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_one_and_two_row_forward_products(fl, fa, fb):
    """Against the oracle within 1e-5 * sum|a||b|, through fp8_scaled_gemm,
    fp8_scaled_gemm_ws (the same kernel, the workspace unused: the same bits),
    fp8_scaled_gemm_amax (max |out| bit-identical) and
    fp8_scaled_gemm_accumulate (old + product)."""
    rng = np.random.default_rng(zlib.crc32(f"gemv {fa} {fb}".encode()))
    for (M, N, K) in GEMV_SHAPES:
        a8, b8 = operands(rng, "fwd", M, N, K, fa, fb)
        ba, bb = (int(v) for v in rng.integers(-12, 20, 2))
        say("gemm one or two rows", "fmts", fa, fb, "MNK", M, N, K)
        A, B, BA, BB = u8_dev(a8), u8_dev(b8), i32_dev(ba), i32_dev(bb)
        got = fl.scaled_gemm(fl.OP_FWD, A, fa, BA, B, fb, BB).cpu().numpy()
        ref, bound = oracle.gemm_fwd(a8, fa, ba, b8, fb, bb)
        check_gemm(got, ref, bound, f"rows {M}x{N}x{K} fmts {fa},{fb}")
        nb = fl.gemm_workspace_bytes(fl.OP_FWD, M, N, K)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        got_ws = fl.scaled_gemm(fl.OP_FWD, A, fa, BA, B, fb, BB, workspace=ws).cpu().numpy()
        if M * K <= 65536:   # the vector (or, K = 0, the row) kernel either way: the same bits
            assert np.array_equal(got_ws.view(np.uint32), got.view(np.uint32))
        else:
            check_gemm(got_ws, ref, bound, f"rows {M}x{N}x{K} split")
        amax = torch.empty(1, dtype=torch.float32, device="cuda")
        got_a = fl.scaled_gemm(fl.OP_FWD, A, fa, BA, B, fb, BB, amax=amax).cpu().numpy()
        assert np.array_equal(got_a.view(np.uint32), got.view(np.uint32))
        want_amax = int(np.max(got.view(np.uint32) & 0x7FFFFFFF)) if got.size else 0
        assert int(amax.cpu().numpy().view(np.uint32)[0]) == want_amax
        old = old_buffer(rng, ref.shape, float(np.sqrt(np.mean(ref ** 2))) if ref.size and np.any(ref) else 1.0)
        acc_ref, _ = oracle.gemm_accumulate(0, old, a8, fa, ba, b8, fb, bb)
        out = torch.from_numpy(old.copy()).cuda()
        fl.scaled_gemm_accumulate(fl.OP_FWD, A, fa, BA, B, fb, BB, out)
        check_gemm(out.cpu().numpy(), acc_ref, bound, f"rows accumulate {M}x{N}x{K}",
                   extra=2.0 ** -24 * np.abs(acc_ref))


# Forward products of 1 to 64 rows whose contraction is a multiple of 256 run
# in the row-streaming MFMA kernel: stages of 256 contraction bytes over 32
# weight rows through LDS DMA, each workgroup starting at its own stage and
# wrapping, eight waves' partial sums added in a fixed order.  One row block
# (1 to 32 rows; over 768 or more column tiles a two-stage ring up to 24 rows
# and two column tiles per workgroup from 25, three stages otherwise) and two
# (33 to 64; over 768 or more column tiles two of them per workgroup in two
# stages), ragged and small column counts, one stage
# (K = 256), 43 stages (K = 11008) and long contractions, K = 0, a contraction
# the kernel does not take (K % 256 != 0: the tiled kernels), 65 rows (the
# tiled kernels).
ROWS_SHAPES = [(1, 4103, 8192), (2, 96, 32768), (3, 1000, 256), (8, 33, 11008), (17, 4103, 2048),
               (2, 24600, 512), (8, 28672, 256), (24, 24576, 256), (25, 24600, 256),
               (32, 24600, 512), (40, 24600, 512), (64, 24576, 256),
               (32, 96, 28672), (31, 1, 512), (33, 1000, 256), (48, 77, 11008), (64, 1000, 8192),
               (5, 40, 0), (64, 40, 0), (8, 300, 320), (65, 64, 512)]


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("mfma", ["auto", "f16", "bf16"])
def test_few_row_forward_products(fl, monkeypatch, fa, fb, mfma):
    """Against the oracle within 1e-5 * sum|a||b|, through fp8_scaled_gemm,
    fp8_scaled_gemm_ws (the same kernel, the workspace unused: the same bits),
    fp8_scaled_gemm_amax (max |out| bit-identical) and
    fp8_scaled_gemm_accumulate (old + product)."""
    if mfma != "auto":
        monkeypatch.setenv("FP8LIN_EXACT_MFMA", mfma)
    else:
        monkeypatch.delenv("FP8LIN_EXACT_MFMA", raising=False)
    rng = np.random.default_rng(zlib.crc32(f"rows {fa} {fb} {mfma}".encode()))
    for (M, N, K) in ROWS_SHAPES:
        a8, b8 = operands(rng, "fwd", M, N, K, fa, fb)
        ba, bb = (int(v) for v in rng.integers(-12, 20, 2))
        say("gemm few rows", "fmts", fa, fb, "mfma", mfma, "MNK", M, N, K)
        A, B, BA, BB = u8_dev(a8), u8_dev(b8), i32_dev(ba), i32_dev(bb)
        got = fl.scaled_gemm(fl.OP_FWD, A, fa, BA, B, fb, BB).cpu().numpy()
        ref, bound = oracle.gemm_fwd(a8, fa, ba, b8, fb, bb)
        check_gemm(got, ref, bound, f"few rows {M}x{N}x{K} fmts {fa},{fb} {mfma}")
        nb = fl.gemm_workspace_bytes(fl.OP_FWD, M, N, K)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        got_ws = fl.scaled_gemm(fl.OP_FWD, A, fa, BA, B, fb, BB, workspace=ws).cpu().numpy()
        if K % 256 == 0 and M <= 64:   # the row kernel either way: the same bits
            assert np.array_equal(got_ws.view(np.uint32), got.view(np.uint32))
        else:
            check_gemm(got_ws, ref, bound, f"few rows {M}x{N}x{K} split")
        amax = torch.empty(1, dtype=torch.float32, device="cuda")
        got_a = fl.scaled_gemm(fl.OP_FWD, A, fa, BA, B, fb, BB, amax=amax).cpu().numpy()
        assert np.array_equal(got_a.view(np.uint32), got.view(np.uint32))
        want_amax = int(np.max(got.view(np.uint32) & 0x7FFFFFFF)) if got.size else 0
        assert int(amax.cpu().numpy().view(np.uint32)[0]) == want_amax
        old = old_buffer(rng, ref.shape, float(np.sqrt(np.mean(ref ** 2))) if ref.size and np.any(ref) else 1.0)
        acc_ref, _ = oracle.gemm_accumulate(0, old, a8, fa, ba, b8, fb, bb)
        out = torch.from_numpy(old.copy()).cuda()
        fl.scaled_gemm_accumulate(fl.OP_FWD, A, fa, BA, B, fb, BB, out)
        check_gemm(out.cpu().numpy(), acc_ref, bound, f"few rows accumulate {M}x{N}x{K}",
                   extra=2.0 ** -24 * np.abs(acc_ref))


def test_one_row_products_with_nan_and_inf_codes(fl):
    """The vector kernel's (2 rows, K = 2064) and the row kernel's (1, 8 and
    40 rows, K = 2048) IEEE arithmetic on NaN codes and E5M2 infinities, as
    the tiled kernels' (R19): NaN where a term is NaN, inf * 0 or inf - inf,
    that infinity where one infinite term has no opposite."""
    rng = np.random.default_rng(zlib.crc32(b"gemv specials"))
    for (fa, fb), (M, K) in zip(PAIRS * 4, [(2, 2064)] * 4 + [(1, 2048)] * 4 + [(8, 2048)] * 4 + [(40, 2048)] * 4):
        a8, b8 = operands(rng, "fwd", M, 300, K, fa, fb)
        a8 = plant_specials(rng, a8, fa, K)
        b8 = plant_specials(rng, b8, fb, K)
        say("gemm few rows, specials", "rows", M, "fmts", fa, fb)
        got = fl.scaled_gemm(fl.OP_FWD, u8_dev(a8), fa, i32_dev(2), u8_dev(b8), fb, i32_dev(-1)).cpu().numpy()
        ref, bound = oracle.gemm_fwd(a8, fa, 2, b8, fb, -1)
        check_gemm(got, ref, bound, f"rows specials fmts {fa},{fb}")


ACC_SHAPES = [(300, 520, 392), (64, 64, 0), (257, 129, 1000), (33, 700, 130), (512, 512, 128),
              (260, 300, 17)]
OP_OF = {"fwd": 0, "dgrad": 1, "wgrad": 2}


def old_buffer(rng, shape, scale):
    """What an accumulation buffer may hold: values of the product's size,
    exact zeros of both signs, and a few far larger ones."""
    old = (rng.standard_normal(shape) * scale).astype(np.float32)
    flat = old.reshape(-1)
    if flat.size:
        idx = rng.choice(flat.size, min(flat.size, 40), replace=False)
        flat[idx[:10]] = 0.0
        flat[idx[10:20]] = -0.0
        flat[idx[20:]] *= 1e4
    return old


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_accumulate_into_the_output(fl, tile, which, fa, fb):
    """fp8_scaled_gemm_accumulate: out = old + product, one fp32 addition per
    output.  Against the oracle's old + exact product (float64):
    |gpu - ref| <= 1e-5 * bound + 2^-24 * |ref| (the addition's rounding);
    then a second product added on top of the first result (two
    micro-batches) against old + product 1 + product 2, within both
    products' bounds and both additions' roundings.  The kernels, tile sizes
    and ragged edges are those of the plain products."""
    rng = np.random.default_rng(zlib.crc32(f"accumulate {which} {fa} {fb}".encode()))
    op = OP_OF[which]
    for (M, N, K) in ACC_SHAPES:
        a8, b8 = operands(rng, which, M, N, K, fa, fb)
        c8, d8 = operands(rng, which, M, N, K, fa, fb)
        ba, bb = (int(v) for v in rng.integers(-12, 20, 2))
        y1, bound1 = reference(which, a8, fa, ba, b8, fb, bb)
        y2, bound2 = reference(which, c8, fa, ba, d8, fb, bb)
        scale = float(np.sqrt(np.mean(y1 ** 2))) if y1.size and np.any(y1) else 1.0
        old = old_buffer(rng, y1.shape, scale)
        ref1, _ = oracle.gemm_accumulate(op, old, a8, fa, ba, b8, fb, bb)
        say("gemm accumulate", which, "tile", tile, "fmts", fa, fb, "MNK", M, N, K)
        out = torch.from_numpy(old.copy()).cuda()
        BA, BB = i32_dev(ba), i32_dev(bb)
        fl.scaled_gemm_accumulate(op, u8_dev(a8), fa, BA, u8_dev(b8), fb, BB, out)
        got1 = out.cpu().numpy()
        check_gemm(got1, ref1, bound1, f"accumulate {which} {M}x{N}x{K} fmts {fa},{fb} tile {tile}",
                   extra=2.0 ** -24 * np.abs(ref1))
        if K == 0:   # old + 0: the buffer itself, -0 turned to +0
            assert np.array_equal(got1, old + np.float32(0.0))
            assert not np.any(np.signbit(got1) & (got1 == 0))
        fl.scaled_gemm_accumulate(op, u8_dev(c8), fa, BA, u8_dev(d8), fb, BB, out)
        ref2 = ref1 + y2
        check_gemm(out.cpu().numpy(), ref2, bound1 + bound2, f"accumulate twice {which} {M}x{N}x{K}",
                   extra=2.0 ** -24 * (np.abs(ref1) + np.abs(ref2)) * (1 + 2.0 ** -20))


@pytest.mark.parametrize("tile_size", ["128", "256"])
def test_accumulate_native_arithmetic(fl, monkeypatch, tile_size):
    """The same through the native FP8 MFMA, against its window bound plus the
    addition's rounding (forward and weight gradient, each pipelined tile)."""
    monkeypatch.setenv("FP8LIN_GEMM_TILE", tile_size)
    rng = np.random.default_rng(zlib.crc32(f"accumulate native {tile_size}".encode()))
    for which, (M, N, K) in (("fwd", (300, 520, 392)), ("wgrad", (512, 512, 128))):
        fa = fb = E4M3
        a8, b8 = operands(rng, which, M, N, K, fa, fb)
        ba, bb = 2, -3
        y, _ = reference(which, a8, fa, ba, b8, fb, bb)
        old = old_buffer(rng, y.shape, float(np.sqrt(np.mean(y ** 2))))
        op = OP_OF[which]
        ref, _ = oracle.gemm_accumulate(op, old, a8, fa, ba, b8, fb, bb)
        av, bv = operand_values(which, oracle.decode_fp8(a8, fa), oracle.decode_fp8(b8, fb))
        nb = native_bound(av, bv, -(ba + bb))
        say("gemm accumulate native", which, "MNK", M, N, K)
        out = torch.from_numpy(old.copy()).cuda()
        fl.scaled_gemm_accumulate(op, u8_dev(a8), fa, i32_dev(ba), u8_dev(b8), fb, i32_dev(bb), out,
                                  math=fl.MATH_NATIVE_FP8)
        check_gemm(out.cpu().numpy(), ref, nb, f"accumulate native {which} {M}x{N}x{K}", rel=1.0,
                   extra=2.0 ** -24 * np.abs(ref))


def plant_specials(rng, codes, fmt, contraction):
    """Put NaN codes (both signs; and for E5M2 the other NaN codes and both
    infinities) at random places of an operand, about one per three
    contraction lines, so some outputs are finite and some are not."""
    flat = codes.reshape(-1)
    if flat.size == 0 or contraction == 0:
        return codes
    specials = np.array([0x7F, 0xFF] + ([0x7C, 0xFC, 0x7D, 0xFE] if fmt == E5M2 else []), dtype=np.uint8)
    n = max(1, flat.size // (3 * contraction))
    idx = rng.choice(flat.size, n, replace=False)
    flat[idx] = rng.choice(specials, n)
    return codes


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_nan_and_inf_codes(fl, tile, which, fa, fb):
    """NaN codes as the cast emits them for NaN inputs (0x7F / 0xFF) and the
    E5M2 infinities (which a caller's codes may hold) in the operands: an
    output whose terms hold a NaN, inf * 0 or inf - inf is NaN, one with an
    infinite term otherwise that infinity, as the oracle's IEEE fp64 sum gives;
    the other outputs stay within the bound."""
    rng = np.random.default_rng(zlib.crc32(f"specials {which} {fa} {fb}".encode()))
    for (M, N, K) in [(300, 520, 392), (257, 129, 1000), (512, 512, 128), (33, 700, 130), (260, 300, 17)]:
        a8, b8 = operands(rng, which, M, N, K, fa, fb)
        contraction = {"fwd": K, "dgrad": N, "wgrad": M}[which]
        a8 = plant_specials(rng, a8, fa, contraction)
        b8 = plant_specials(rng, b8, fb, contraction)
        ba, bb = (int(v) for v in rng.integers(-12, 20, 2))
        say("specials", which, "tile", tile, "fmts", fa, fb, "MNK", M, N, K)
        got = run(fl, which, a8, fa, ba, b8, fb, bb)
        ref, bound = reference(which, a8, fa, ba, b8, fb, bb)
        nonfinite = ~np.isfinite(ref)
        assert 0 < nonfinite.sum() < ref.size, (which, M, N, K)   # both kinds present
        check_gemm(got, ref, bound, f"specials {which} {M}x{N}x{K} fmts {fa},{fb} tile {tile}")


# ba + bb from deep underflow to overflow: 2^-(ba+bb) takes the outputs into
# fp32's subnormal range and below (+150, +140), to its smallest normals
# (+126), and beyond its largest finite value (-128, -150)
UNSCALES = [(75, 75), (100, 40), (63, 63), (-64, -64), (-75, -75), (-200, 221)]


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_unscale_into_fp32_subnormal_underflow_and_overflow(fl, tile, which):
    """The unscale's ldexp rounds once where the result is an fp32 subnormal
    (to zero below half the smallest one) and gives the infinity of the
    result's sign beyond fp32's largest finite value: within the bound plus
    half the subnormal spacing, or that infinity (check_gemm)."""
    rng = np.random.default_rng(zlib.crc32(f"unscale {which}".encode()))
    for (M, N, K) in [(300, 520, 392), (512, 512, 128), (260, 300, 17)]:
        for fa, fb in [(E4M3, E4M3), (E5M2, E4M3)]:
            a8, b8 = operands(rng, which, M, N, K, fa, fb)
            for ba, bb in UNSCALES:
                say("unscale", which, "tile", tile, "fmts", fa, fb, "MNK", M, N, K, "biases", ba, bb)
                got = run(fl, which, a8, fa, ba, b8, fb, bb)
                ref, bound = reference(which, a8, fa, ba, b8, fb, bb)
                check_gemm(got, ref, bound, f"unscale {ba}+{bb} {which} {M}x{N}x{K} tile {tile}")
                sub = (got != 0) & (np.abs(got) < 2.0 ** -126)
                if ba + bb >= 140:      # the range is reached: subnormal outputs
                    assert sub.any()
                if ba + bb <= -128:     # and here some really overflow
                    assert np.isinf(got).any()


def test_unscale_range_in_split_products(fl):
    """The same extremes through the split products' ordered reduction."""
    rng = np.random.default_rng(zlib.crc32(b"unscale split"))
    for op, (M, N, K) in ((0, (128, 256, 4096)), (1, (96, 6400, 80)), (2, (3200, 128, 256))):
        which = ("fwd", "dgrad", "wgrad")[op]
        fa, fb = (E4M3, E4M3) if op == 0 else (E5M2, E4M3)
        a8, b8 = operands(rng, which, M, N, K, fa, fb)
        nbytes = fl.gemm_workspace_bytes(op, M, N, K)
        assert nbytes > 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        for ba, bb in UNSCALES:
            say("unscale split", which, M, N, K, "biases", ba, bb)
            got = fl.scaled_gemm(op, u8_dev(a8), fa, i32_dev(ba), u8_dev(b8), fb, i32_dev(bb),
                                 workspace=ws).cpu().numpy()
            ref, bound = reference(which, a8, fa, ba, b8, fb, bb)
            check_gemm(got, ref, bound, f"split unscale {ba}+{bb} {which} {M}x{N}x{K}")


def test_all_positive_long_contraction_stays_within_bound(fl):
    """Accumulation stress: same-sign products over K = 28672 (the longest
    contraction in the workloads), where fp32 rounding adds up fastest."""
    rng = np.random.default_rng(99)
    M, N, K = 96, 80, 28672
    x8 = rng.integers(0x30, 0x60, (M, K), dtype=np.uint8)   # positive E4M3 codes
    w8 = rng.integers(0x30, 0x60, (N, K), dtype=np.uint8)
    say("positive long K", M, N, K)
    got = run(fl, "fwd", x8, E4M3, 0, w8, E4M3, 0)
    ref, bound = oracle.gemm_fwd(x8, E4M3, 0, w8, E4M3, 0)
    worst = check_gemm(got, ref, bound, "all-positive fwd K=28672")
    print("worst err/bound", worst)


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3)])
def test_native_fp8_math_within_its_bound(fl, tile, which, fa, fb):
    """The opt-in native FP8 MFMA arithmetic (fp8_scaled_gemm, FP8_GEMM_NATIVE_FP8)
    within the bound of its measured summation (tests/mfma_bound.py: each
    64-product instruction keeps the bits down to 2^(E - 13) below its largest
    product, plus one fp32 rounding per instruction), on random codes and on
    N(0, 1)-valued codes; a wrong product in each group falls outside it."""
    rng = np.random.default_rng(zlib.crc32(f"native {which} {fa} {fb}".encode()))
    op = {"fwd": fl.OP_FWD, "dgrad": fl.OP_DGRAD, "wgrad": fl.OP_WGRAD}[which]
    worst = 0.0
    for (M, N, K) in [(300, 520, 392), (257, 129, 1000), (512, 512, 128)]:
        for data in ("codes", "normal"):
            if data == "codes":
                a8, b8 = operands(rng, which, M, N, K, fa, fb)
            else:
                a8, b8 = normal_operands(rng, which, M, N, K, fa, fb)
            say("native fp8", which, "tile", tile, "fmts", fa, fb, "MNK", M, N, K, data)
            got = fl.scaled_gemm(op, u8_dev(a8), fa, i32_dev(3), u8_dev(b8), fb, i32_dev(-2),
                                 math=fl.MATH_NATIVE_FP8).cpu().numpy()
            ref, mag = reference(which, a8, fa, 3, b8, fb, -2)
            a, b = operand_values(which, oracle.decode_fp8(a8, fa), oracle.decode_fp8(b8, fb))
            bound = native_bound(a, b, -1)
            check_gemm(got, ref, bound, f"native {which} {M}x{N}x{K} {data}", rel=1.0)
            worst = max(worst, float(np.max(np.abs(got - ref) / np.where(mag > 0, mag, 1.0))))
    print(f"native fp8 {which}: worst err/sum|ab| {worst:.3e}")


def normal_operands(rng, which, M, N, K, fa, fb):
    """Codes of N(0, 1) values scaled so the largest lands near the format's
    top (the AMAX scaling of the workloads)."""
    def codes(shape, fmt):
        dt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
        v = rng.standard_normal(shape) * (448.0 if fmt == E4M3 else 57344.0) / 5.0
        v = np.clip(v, -448.0 if fmt == E4M3 else -57344.0, 448.0 if fmt == E4M3 else 57344.0)
        return torch.tensor(v, dtype=torch.float32).to(dt).view(torch.uint8).numpy()
    if which == "fwd":
        return codes((M, K), fa), codes((N, K), fb)
    if which == "dgrad":
        return codes((M, N), fa), codes((N, K), fb)
    return codes((M, N), fa), codes((M, K), fb)


def _sample_positions(rng, rows, cols, count=65536):
    r = rng.integers(0, rows, count)
    c = rng.integers(0, cols, count)
    # plus the first and the last 256 x 256 output tiles
    t = np.arange(256)
    fr, fc = np.meshgrid(t[t < rows], t[t < cols], indexing="ij")
    lr, lc = np.meshgrid(np.arange(max(rows - 256, 0), rows), np.arange(max(cols - 256, 0), cols), indexing="ij")
    return (np.concatenate([r, fr.ravel(), lr.ravel()]).astype(np.int64),
            np.concatenate([c, fc.ravel(), lc.ravel()]).astype(np.int64))


def _quantized(w, name, cache):
    if name not in cache:
        t = w.tensor(name)
        words = synth.bf16_words(synth.workload_tensor(w, name))
        a, b, codes = oracle.quantize(words, t.fmt, t.margin)
        cache[name] = (codes, b, t.fmt)
    return cache[name]


@pytest.mark.parametrize("wl", [1, 2, 3, 4, 5])
def test_workload_products(fl, wl):
    """Every product of a workload at its full size, in the launch configuration
    the benchmark uses; the oracle checks every output for the two small
    workloads and 65536 random outputs plus the first and last 256x256 tiles
    of each product for the others."""
    w = synth.WORKLOADS[wl]
    rng = np.random.default_rng(wl)
    cache = {}
    full = wl <= 2
    for l in w.linears:
        x8, bx, fx = _quantized(w, l.x, cache)
        wt8, bw, fw = _quantized(w, l.w, cache)
        if l.dy:
            dy8, bdy, fdy = _quantized(w, l.dy, cache)
        for which in l.passes:
            if which == "fwd":
                a8, fa, ba, b8, fb, bb = x8, fx, bx, wt8, fw, bw
                shape = (l.M, l.N)
            elif which == "dgrad":
                a8, fa, ba, b8, fb, bb = dy8, fdy, bdy, wt8, fw, bw
                shape = (l.M, l.K)
            else:
                a8, fa, ba, b8, fb, bb = dy8, fdy, bdy, x8, fx, bx
                shape = (l.N, l.K)
            say("workload", wl, l.name, which, "out", shape)
            got = run(fl, which, a8, fa, ba, b8, fb, bb)
            assert got.shape == shape
            if full:
                ref, bound = reference(which, a8, fa, ba, b8, fb, bb)
                check_gemm(got, ref, bound, f"wl{wl} {l.name} {which}")
            else:
                rows, cols = _sample_positions(rng, *shape)
                at = {"fwd": oracle.gemm_fwd_at, "dgrad": oracle.gemm_dgrad_at,
                      "wgrad": oracle.gemm_wgrad_at}[which]
                ref, bound = at(a8, fa, ba, b8, fb, bb, rows, cols)
                check_gemm(got[rows, cols], ref, bound, f"wl{wl} {l.name} {which}")
            del got


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_epilogue_amax_is_the_amax_of_the_output(fl, tile, which):
    """fp8_scaled_gemm_amax: the product's output is the same as without it,
    and the amax its epilogue folds is bit-identical to max |out| of that
    output (and to fp8_amax over it).  An empty product leaves amax 0."""
    rng = np.random.default_rng(77)
    op = {"fwd": fl.OP_FWD, "dgrad": fl.OP_DGRAD, "wgrad": fl.OP_WGRAD}[which]
    for (M, N, K) in [(300, 520, 392), (257, 129, 1000), (512, 512, 128), (64, 64, 0), (1, 17, 1), (0, 8, 8)]:
        a8, b8 = operands(rng, which, M, N, K, E5M2, E4M3)
        A, B, BA, BB = u8_dev(a8), u8_dev(b8), i32_dev(3), i32_dev(-2)
        say("epilogue amax", which, "tile", tile, "MNK", M, N, K)
        plain = fl.scaled_gemm(op, A, E5M2, BA, B, E4M3, BB)
        amax = torch.full((1,), 12345.0, dtype=torch.float32, device="cuda")
        got = fl.scaled_gemm(op, A, E5M2, BA, B, E4M3, BB, amax=amax)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), plain.view(torch.int32))
        bits = got.view(torch.int32).cpu().numpy().astype(np.uint32) & 0x7FFFFFFF
        want = int(bits.max()) if bits.size else 0
        assert int(amax.view(torch.int32).cpu().item()) == want
        if got.numel():
            assert torch.equal(fl.amax(got.reshape(-1)).view(torch.int32), amax.view(torch.int32))


def test_epilogue_amax_drives_the_next_quantisation(fl):
    """Quantising a product's fp32 output with the bias from its epilogue
    amax gives the oracle's codes for that output (amax, bias and cast
    bit-exact, "Proposed method" bullets 1-4)."""
    rng = np.random.default_rng(78)
    M, N, K = 384, 640, 512
    a8, b8 = operands(rng, "fwd", M, N, K, E4M3, E4M3)
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    y = fl.scaled_gemm(fl.OP_FWD, u8_dev(a8), E4M3, i32_dev(4), u8_dev(b8), E4M3, i32_dev(5), amax=amax)
    for fmt in (E4M3, E5M2):
        bias = fl.compute_bias(amax, fmt, 1)
        codes = fl.scale_cast(y.reshape(-1), bias, fmt).cpu().numpy()
        words = y.reshape(-1).view(torch.int32).cpu().numpy().view(np.uint32)
        b = oracle.compute_bias(oracle.amax_bits(words), fmt, 1)
        assert int(bias.cpu().item()) == b
        assert np.array_equal(codes, oracle.scale_cast(words, b, fmt))


# Output shapes whose 256x256 tiling leaves a part-empty last wave, so the
# launch takes a block of whole waves in 256x256 tiles and the rest of the
# rows (row split) or columns (column split) in 128x128 tiles; the sampled
# outputs include every row / column next to the split and the last ones.
SPLIT_SHAPES = [  # (product, output rows, output cols, contraction, expected split)
    ("fwd", 4096, 5120, 128, "columns at 4096"),
    ("dgrad", 4096, 5120, 64, "columns at 4096"),
    ("wgrad", 13824, 5120, 64, "rows at 13056"),
    ("fwd", 4096, 22016, 64, "columns at 20480"),
    ("dgrad", 4096, 13824, 64, "rows at 3584"),
]


@pytest.mark.parametrize("math", ["exact", "native"])
@pytest.mark.parametrize("which,R,C,Kc,split", SPLIT_SHAPES)
def test_two_launch_split_of_the_output(fl, which, R, C, Kc, split, math):
    rng = np.random.default_rng(R + C + Kc)
    fa, fb = (E4M3, E4M3) if which == "fwd" else (E5M2, E4M3)
    # problem sizes (M, N, K) of each product for an R x C output
    M, N, K = {"fwd": (R, C, Kc), "dgrad": (R, Kc, C), "wgrad": (Kc, R, C)}[which]
    a8, b8 = operands(rng, which, M, N, K, fa, fb)
    say("split launch", which, R, C, Kc, split)
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    op = {"fwd": fl.OP_FWD, "dgrad": fl.OP_DGRAD, "wgrad": fl.OP_WGRAD}[which]
    mth = fl.MATH_EXACT if math == "exact" else fl.MATH_NATIVE_FP8
    out = fl.scaled_gemm(op, u8_dev(a8), fa, i32_dev(2), u8_dev(b8), fb, i32_dev(-1), math=mth, amax=am)
    got = out.cpu().numpy()
    at = {"fwd": oracle.gemm_fwd_at, "dgrad": oracle.gemm_dgrad_at, "wgrad": oracle.gemm_wgrad_at}[which]
    b_at = int(split.split()[-1])
    rows = np.concatenate([rng.integers(0, R, 3000), np.repeat(np.arange(R - 3, R), 40)])
    cols = np.concatenate([rng.integers(0, C, 3000), rng.integers(0, C, 120)])
    if split.startswith("rows"):
        band = np.repeat(np.arange(b_at - 8, b_at + 8), 64)
        rows = np.concatenate([rows, band])
        cols = np.concatenate([cols, rng.integers(0, C, band.size)])
    else:
        band = np.repeat(np.arange(b_at - 8, b_at + 8), 64)
        cols = np.concatenate([cols, band])
        rows = np.concatenate([rows, rng.integers(0, R, band.size)])
    ref, bound = at(a8, fa, 2, b8, fb, -1, rows, cols)
    if math == "native":   # the native FP8 MFMA's own bound (test_native_fp8_math_within_its_bound)
        bound = native_bound_at(which, a8, fa, b8, fb, rows, cols, -1)
    rel = 1e-5 if math == "exact" else 1.0
    check_gemm(got[rows, cols], ref, bound, f"split {which} {R}x{C} ({split}) {math}", rel=rel)
    # the epilogue amax covers both launches
    assert int(am.view(torch.int32).item()) & 0xFFFFFFFF == int((got.view(np.uint32) & 0x7FFFFFFF).max())


# Products split along the contraction (fp8_scaled_gemm_ws): outputs of few
# 128 x 128 tiles, contraction lengths split evenly (3200 = 50 stages in two)
# and unevenly (3136 = 49 stages: 25 + 24, the shortest slice allowed), ragged output sides (multiples of 16 where an operand is
# read contraction-major), a single tile split ten ways, and per product one
# shape that is not split (workspace 0).
SPLIT_SHAPES = {
    "fwd": [(128, 256, 4096), (100, 300, 3200), (128, 256, 3136), (16, 48, 6400), (100, 100, 15360),
            (2048, 768, 3072), (1024, 2048, 4096), (2048, 2048, 1024)],
    "dgrad": [(128, 3200, 256), (96, 6400, 80), (2048, 3072, 768), (1024, 4096, 2048), (2048, 1024, 2048)],
    "wgrad": [(3200, 128, 256), (6400, 96, 80), (3072, 2304, 768), (4096, 1024, 2048), (1024, 2048, 2048)],
}
UNSPLIT = {(2048, 2048, 1024), (2048, 1024, 2048), (1024, 2048, 2048)}   # 256 output tiles


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_split_products_against_the_oracle(fl, which):
    """Within the bound of every (M, N, K) and format pair, both exact MFMAs;
    bit-identical on a second call (the slices are added in a fixed order);
    a too small workspace is refused before anything runs."""
    op = {"fwd": fl.OP_FWD, "dgrad": fl.OP_DGRAD, "wgrad": fl.OP_WGRAD}[which]
    rng = np.random.default_rng(4242)
    for si, (M, N, K) in enumerate(SPLIT_SHAPES[which]):
        nbytes = fl.gemm_workspace_bytes(op, M, N, K)
        assert (nbytes == 0) == ((M, N, K) in UNSPLIT), (which, M, N, K, nbytes)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        for fa, fb in PAIRS:
            a8, b8 = operands(rng, which, M, N, K, fa, fb)
            ba, bb = int(rng.integers(-12, 20)), int(rng.integers(-12, 20))
            ref, bound = reference(which, a8, fa, ba, b8, fb, bb)
            A, B, BA, BB = u8_dev(a8), u8_dev(b8), i32_dev(ba), i32_dev(bb)
            for mfma in ("f16", "bf16"):
                os.environ["FP8LIN_EXACT_MFMA"] = mfma
                try:
                    say("split product", which, "shape", M, N, K, "fmts", fa, fb, "mfma", mfma, "ws", nbytes)
                    got = fl.scaled_gemm(op, A, fa, BA, B, fb, BB, workspace=ws)
                    again = fl.scaled_gemm(op, A, fa, BA, B, fb, BB, workspace=ws)
                finally:
                    del os.environ["FP8LIN_EXACT_MFMA"]
                assert torch.equal(got.view(torch.int32), again.view(torch.int32)), (which, M, N, K)
                check_gemm(got.cpu().numpy(), ref, bound, f"split {which} {M}x{N}x{K} {fa}{fb} {mfma}")
        if nbytes > 0:
            with pytest.raises(fl.Fp8Error) as e:
                fl.scaled_gemm(op, A, fa, BA, B, fb, BB, workspace=ws[:nbytes - 16])
            assert e.value.status == -2


def test_split_product_native_fp8_and_unsplit_identity(fl):
    """The native FP8 arithmetic split within its own bound (2^-7 of sum |ab|
    per 64 products, plus fp32 rounding); an unsplit shape with a workspace
    is fp8_scaled_gemm itself, bit for bit."""
    rng = np.random.default_rng(77)
    M, N, K = 128, 512, 4096
    a8, b8 = operands(rng, "fwd", M, N, K, E4M3, E4M3)
    ref, bound = reference("fwd", a8, E4M3, 3, b8, E4M3, 5)
    A, B, BA, BB = u8_dev(a8), u8_dev(b8), i32_dev(3), i32_dev(5)
    nbytes = fl.gemm_workspace_bytes(fl.OP_FWD, M, N, K)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    say("split native", M, N, K)
    got = fl.scaled_gemm(fl.OP_FWD, A, E4M3, BA, B, E4M3, BB, math=fl.MATH_NATIVE_FP8, workspace=ws)
    # the native arithmetic's bound, plus one fp32 rounding per slice added
    splits = nbytes // (M * N * 4)
    a, b = operand_values("fwd", oracle.decode_fp8(a8, E4M3), oracle.decode_fp8(b8, E4M3))
    check_gemm(got.cpu().numpy(), ref, native_bound(a, b, -8, extra=splits), "native split", rel=1.0)
    M, N, K = 2048, 2048, 1024        # 256 output tiles of 128 x 128: not split
    assert fl.gemm_workspace_bytes(fl.OP_FWD, M, N, K) == 0
    a8, b8 = operands(rng, "fwd", M, N, K, E4M3, E4M3)
    A, B = u8_dev(a8), u8_dev(b8)
    plain = fl.scaled_gemm(fl.OP_FWD, A, E4M3, BA, B, E4M3, BB)
    with_ws = fl.scaled_gemm(fl.OP_FWD, A, E4M3, BA, B, E4M3, BB, workspace=ws)
    assert torch.equal(plain.view(torch.int32), with_ws.view(torch.int32))


def _group_case(fl, rng, specs, fa_fb=None):
    """Products (op name, M, N, K[, fa, fb]) with random codes and biases: the
    binding's product tuples, the host codes and biases."""
    prods, host = [], []
    for spec in specs:
        which, M, N, K = spec[:4]
        fa, fb = spec[4:6] if len(spec) > 4 else ((E4M3, E4M3) if which == "fwd" else (E5M2, E4M3))
        a8, b8 = operands(rng, which, M, N, K, fa, fb)
        ba, bb = int(rng.integers(-12, 20)), int(rng.integers(-12, 20))
        op = {"fwd": fl.OP_FWD, "dgrad": fl.OP_DGRAD, "wgrad": fl.OP_WGRAD}[which]
        prods.append((op, u8_dev(a8), fa, i32_dev(ba), u8_dev(b8), fb, i32_dev(bb)))
        host.append((which, a8, fa, ba, b8, fb, bb))
    return prods, host


GROUP_SPECS = [
    # the GPT-111M layer's nine products at 2048 tokens (some split in the group)
    ("fwd", 2048, 2304, 768), ("fwd", 2048, 3072, 768), ("fwd", 2048, 768, 3072),
    ("dgrad", 2048, 2304, 768), ("dgrad", 2048, 3072, 768), ("dgrad", 2048, 768, 3072),
    ("wgrad", 2048, 2304, 768), ("wgrad", 2048, 3072, 768), ("wgrad", 2048, 768, 3072),
    # ragged sides, every format pair, an empty product, one run alone (K = 100)
    ("fwd", 300, 520, 392, E5M2, E5M2), ("fwd", 33, 700, 1280, E4M3, E5M2), ("fwd", 64, 64, 0),
    ("dgrad", 96, 6400, 80, E5M2, E5M2), ("wgrad", 3200, 128, 256, E4M3, E5M2), ("fwd", 130, 70, 100),
    ("fwd", 0, 16, 64),
]


@pytest.mark.parametrize("mfma", ["auto", "f16", "bf16"])
def test_grouped_products(fl, mfma, monkeypatch):
    """fp8_scaled_gemm_group: every product within the oracle's bound; the
    unsplit ones bit-identical to fp8_scaled_gemm (the same accumulation
    order); a second call bit-identical to the first."""
    if mfma != "auto":
        monkeypatch.setenv("FP8LIN_EXACT_MFMA", mfma)
    rng = np.random.default_rng(zlib.crc32(f"group {mfma}".encode()))
    prods, host = _group_case(fl, rng, GROUP_SPECS)
    say("grouped products", len(prods), "mfma", mfma)
    g = fl.GemmGroup(prods)
    assert g.ws_bytes > 0
    outs = [o.clone() for o in g.run()]
    again = g.run()
    torch.cuda.synchronize()
    for (op, A, fa, BA, B, fb, BB), (which, a8, _, ba, b8, _, bb), got, got2 in zip(prods, host, outs, again):
        assert torch.equal(got.view(torch.int32), got2.view(torch.int32)), which
        ref, bound = reference(which, a8, fa, ba, b8, fb, bb)
        check_gemm(got.cpu().numpy(), ref, bound, f"grouped {which} {a8.shape} {b8.shape}")
        single = fl.scaled_gemm(op, A, fa, BA, B, fb, BB)
        same = torch.equal(single.view(torch.int32), got.view(torch.int32))
        contraction = {"fwd": a8.shape[1], "dgrad": a8.shape[1], "wgrad": a8.shape[0]}[which]
        if contraction in (768, 392, 0, 100):   # never split in this group, whatever the MFMA
            assert same, (which, a8.shape, b8.shape)


def test_grouped_products_of_a_small_batch(fl):
    """A decode-shaped group (8 tokens through a 16 MiB weight and a 32 MiB
    one, 2 tokens through one with K not a multiple of 256, and a small
    weight): the large-weight products run alone in the small-row kernels,
    bit-identical to fp8_scaled_gemm; the small one stays grouped; every
    product against the oracle."""
    rng = np.random.default_rng(zlib.crc32(b"group small batch"))
    specs = [("fwd", 8, 8192, 2048), ("fwd", 8, 4096, 8192), ("fwd", 2, 65536, 272), ("fwd", 8, 768, 768)]
    prods, host = _group_case(fl, rng, specs)
    say("grouped small batch", len(prods))
    outs = fl.scaled_gemm_group(prods)
    for (op, A, fa, BA, B, fb, BB), (which, a8, _, ba, b8, _, bb), got in zip(prods, host, outs):
        ref, bound = reference(which, a8, fa, ba, b8, fb, bb)
        check_gemm(got.cpu().numpy(), ref, bound, f"grouped small batch {a8.shape} {b8.shape}")
        single = fl.scaled_gemm(op, A, fa, BA, B, fb, BB)
        if b8.size >= 1 << 24:   # alone in the small-row kernel: the same call
            assert torch.equal(single.view(torch.int32), got.view(torch.int32)), b8.shape


def test_grouped_products_native_arithmetic(fl):
    """The native FP8 arithmetic through the group, within its own bound
    (tests/mfma_bound.py; one extra fp32 rounding per slice added)."""
    rng = np.random.default_rng(zlib.crc32(b"group native"))
    specs = [("fwd", 2048, 768, 3072), ("fwd", 300, 520, 392), ("dgrad", 512, 768, 256)]
    prods, host = _group_case(fl, rng, specs)
    say("grouped native", len(prods))
    outs = fl.scaled_gemm_group(prods, math=fl.MATH_NATIVE_FP8)
    for (which, a8, fa, ba, b8, fb, bb), got in zip(host, outs):
        ref, _ = reference(which, a8, fa, ba, b8, fb, bb)
        a, b = operand_values(which, oracle.decode_fp8(a8, fa), oracle.decode_fp8(b8, fb))
        check_gemm(got.cpu().numpy(), ref, native_bound(a, b, -(ba + bb), extra=16),
                   f"grouped native {which}", rel=1.0)


def test_grouped_products_of_a_workload_step(fl):
    """The GPT-111M layer's nine products from the workload's own quantised
    tensors (the oracle's codes), grouped, against the oracle."""
    w = synth.WORKLOADS[2]
    cache = {}
    prods, host = [], []
    op_of = {"fwd": fl.OP_FWD, "dgrad": fl.OP_DGRAD, "wgrad": fl.OP_WGRAD}
    for l in w.linears:
        for which in l.passes:
            an, bn = {"fwd": (l.x, l.w), "dgrad": (l.dy, l.w), "wgrad": (l.dy, l.x)}[which]
            a8, ba, fa = _quantized(w, an, cache)
            b8, bb, fb = _quantized(w, bn, cache)
            prods.append((op_of[which], u8_dev(a8), fa, i32_dev(ba), u8_dev(b8), fb, i32_dev(bb)))
            host.append((which, a8, fa, ba, b8, fb, bb))
    say("grouped workload 2")
    outs = fl.scaled_gemm_group(prods)
    for (which, a8, fa, ba, b8, fb, bb), got in zip(host, outs):
        ref, bound = reference(which, a8, fa, ba, b8, fb, bb)
        check_gemm(got.cpu().numpy(), ref, bound, f"grouped wl2 {which}")
