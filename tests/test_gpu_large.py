"""Tensors past 2^31 elements or bytes: every kernel family at a size where a
32-bit offset would wrap, checked by properties that hold at any size (a
planted maximum decides the amax exactly) and against the oracle at sampled
positions (windows of the cast straddling element 2^31; products and SwiGLU
rows past the 2^31st byte or element).  Inputs are generated on the device.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_gemm, i32_dev, need_gpu, say, words_of

pytestmark = pytest.mark.gpu
E4M3, E5M2 = 0, 1
BIG = (1 << 31) + 4099


@pytest.fixture(scope="module")
def fl():
    return need_gpu()


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_amax_and_cast_past_2_31_elements(fl, dtype):
    n = BIG if dtype == torch.bfloat16 else (1 << 31) + 517
    say("large amax/cast", dtype, n)
    torch.manual_seed(1)
    x = torch.randn(n, dtype=dtype, device="cuda")
    for pos, val in ((5, -1000.0), (n - 3, 1000.0)):
        keep = x[pos].clone()
        x[pos] = val
        a = fl.amax(x)
        assert a.item() == 1000.0, (pos, a.item())        # |randn| is far below 1000
        x[pos] = keep
    codes, bias, amax = fl.quantize(x, E4M3, 0)
    a_bits = int(words_of(amax)[0])
    b = int(bias.item())
    assert b == oracle.compute_bias(a_bits, E4M3, 0)
    for lo in (0, (1 << 31) - 40000, n - 70000):
        hi = min(n, lo + 70000)
        words = words_of(x[lo:hi])
        got = codes[lo:hi].cpu().numpy()
        assert np.array_equal(got, oracle.scale_cast(words, b, E4M3)), (dtype, lo)
    # the cast with its amax folded in (a main cast over 2^31 elements, then
    # the last block over the stretch) and delayed scaling in one call: the
    # same codes, bit for bit, and the same amax
    say("large fused cast + amax", dtype, n)
    am = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    fused = fl.scale_cast(x, bias, E4M3, amax=am)
    assert torch.equal(fused, codes) and int(words_of(am)[0]) == a_bits
    del fused
    prev = amax.clone()
    delayed, db = fl.quantize_delayed(x, E4M3, prev, 0)
    assert int(db.item()) == b and torch.equal(delayed, codes) and int(words_of(prev)[0]) == a_bits
    del delayed
    for pos in (n - 5, (1 << 31) - 100000):   # in the last block's stretch, and in the main cast
        keep = x[pos].clone()
        x[pos] = -1000.0
        am.fill_(7.0)
        fl.scale_cast(x, bias, E4M3, out=codes, amax=am)
        assert am.item() == 1000.0, (dtype, pos, am.item())
        x[pos] = keep
    del x, codes
    free()


def test_swiglu_past_2_31_elements(fl):
    rows, f = 32768, 32800                 # h: 2.15e9 floats; dh: 2.15e9 bf16 values
    say("large swiglu", rows, f)
    torch.manual_seed(2)
    h = torch.randn(rows, 2 * f, device="cuda").mul_(3)
    h[rows - 1, f - 1] = 64.0               # g: silu(64) = 64 in fp32
    h[rows - 1, 2 * f - 1] = 64.0           # u: a = 4096 (a bf16 value), far above the rest
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    a = fl.swiglu_fwd(h, amax=am)
    assert am.item() == 4096.0
    da = torch.randn(rows, f, device="cuda").mul_(1e-3)
    dam = torch.empty(1, dtype=torch.float32, device="cuda")
    dh = fl.swiglu_bwd(h, da, amax=dam)
    assert int(words_of(dam)[0]) == int(words_of(dh.abs().max().float().reshape(1))[0])
    for r in (0, rows // 2, rows - 2, rows - 1):
        hr = h[r:r + 1].cpu().numpy()
        dr = da[r:r + 1].cpu().numpy()
        ea = oracle.swiglu_fwd(hr)
        got = a[r:r + 1].float().cpu().numpy()
        assert np.all(np.abs(got - ea) <= 2.0 ** -8 * np.abs(ea) * (1 + 2.0 ** -10) + 2.0 ** -133), r
        ed = oracle.swiglu_bwd(hr, dr)
        g, u = hr[:, :f].astype(np.float64), hr[:, f:].astype(np.float64)
        slack = np.concatenate([2.0 ** -20 * np.abs(dr * u) * (1 + np.abs(g)), np.zeros_like(g)], axis=1)
        gd = dh[r:r + 1].float().cpu().numpy()
        assert np.all(np.abs(gd - ed) <= 2.0 ** -8 * np.abs(ed) * (1 + 2.0 ** -10) + 2.0 ** -133 + slack), r
    del h, a, da, dh
    free()


def random_codes(shape, seed):
    """E4M3 / E5M2 codes without NaN: magnitudes 0..0x7A, random sign."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    mag = torch.randint(0, 0x7B, shape, dtype=torch.uint8, device="cuda", generator=g)
    sign = torch.randint(0, 2, shape, dtype=torch.uint8, device="cuda", generator=g) << 7
    return mag | sign


@pytest.mark.parametrize("K", [32768, 32776])   # pipelined kernel; general kernel (K % 64 != 0)
def test_products_past_2_31_operand_bytes(fl, K):
    M, N = 65600, 512                        # X8: M x K > 2^31 bytes
    say("large products", M, N, K)
    x8 = random_codes((M, K), 11)
    w8 = random_codes((N, K), 12)
    dy8 = random_codes((M, N), 13)
    b0, b1 = i32_dev(3), i32_dev(-2)
    y = fl.scaled_gemm(fl.OP_FWD, x8, E4M3, b0, w8, E4M3, b1)
    dx = fl.scaled_gemm(fl.OP_DGRAD, dy8, E5M2, b0, w8, E4M3, b1)
    dw = fl.scaled_gemm(fl.OP_WGRAD, dy8, E5M2, b0, x8, E4M3, b1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    x8h, w8h, dy8h = x8.cpu().numpy(), w8.cpu().numpy(), dy8.cpu().numpy()
    rows = np.concatenate([rng.integers(0, M, 200), M - 1 - rng.integers(0, 64, 56)])
    cols = rng.integers(0, N, rows.size)
    ref, bound = oracle.gemm_fwd_at(x8h, E4M3, 3, w8h, E4M3, -2, rows, cols)
    check_gemm(y.cpu().numpy()[rows, cols], ref, bound, f"fwd M={M} K={K}")
    kc = np.concatenate([rng.integers(0, K, 200), K - 1 - rng.integers(0, 64, 56)])
    ref, bound = oracle.gemm_dgrad_at(dy8h, E5M2, 3, w8h, E4M3, -2, rows, kc)
    check_gemm(dx[torch.from_numpy(rows).cuda(), torch.from_numpy(kc).cuda()].cpu().numpy(),
               ref, bound, f"dgrad M={M} K={K}")
    ref, bound = oracle.gemm_wgrad_at(dy8h, E5M2, 3, x8h, E4M3, -2, cols, kc)
    check_gemm(dw.cpu().numpy()[cols, kc], ref, bound, f"wgrad M={M} K={K}")
    del x8, w8, dy8, y, dx, dw
    free()


@pytest.mark.parametrize("M,N", [(2, (1 << 26) - 16), (1, (1 << 26) + 16)])
def test_few_row_products_at_the_largest_vector_grid(fl, M, N):
    """A dispatch counts its lanes in 32 bits.  The one-or-two-row vector
    kernel launches 1024 lanes per 16 columns, so it takes at most 2^26 - 16
    columns (its largest grid, 2^32 - 1024 lanes) and hands 2^26 + 16 to the
    tiled kernels (here the general one: K = 16).  Sampled outputs, the last
    columns among them, against the oracle.  (The row kernel's limit, 2^28
    columns, would need a weight of 68 GB or more.)"""
    K = 16
    say("few-row products at the largest grid", M, N, K)
    x8 = random_codes((M, K), 21)
    w8 = random_codes((N, K), 22)
    b0, b1 = i32_dev(4), i32_dev(-3)
    y = fl.scaled_gemm(fl.OP_FWD, x8, E4M3, b0, w8, E4M3, b1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N)
    cols = np.concatenate([rng.integers(0, N, 200), N - 1 - np.arange(56)])
    rows = rng.integers(0, M, cols.size)
    idx = torch.from_numpy(cols).cuda()
    wsub = w8[idx].cpu().numpy()             # the sampled weight rows only
    ref, bound = oracle.gemm_fwd_at(x8.cpu().numpy(), E4M3, 4, wsub, E4M3, -3, rows, np.arange(cols.size))
    got = y[torch.from_numpy(rows).cuda(), idx].cpu().numpy()
    check_gemm(got, ref, bound, f"few rows M={M} N={N}")
    del x8, w8, y
    free()
