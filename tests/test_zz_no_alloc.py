"""fp8_scaled_gemm_noalloc, the product for callers that cannot allocate: its
split workspace is the library's static per-GPU scratch.  Checked through the
C ABI against fp8_scaled_gemm_ws with a caller's workspace (the same kernels
and plan, so the same bits) and against the oracle's bound
(|gpu - oracle| <= 1e-5 * 2^-(ba+bb) * sum |a||b|, "Training and inference of
large language models using 8-bit floating point", review page, "Proposed
method", bullet 3), on consecutive calls whose second input is smaller, so
the second call reads a scratch the first one left filled."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_gemm, i32_dev, need_gpu, say, u8_dev

pytestmark = pytest.mark.gpu
E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def fl():
    return need_gpu()


def _codes(rng, shape, fmt):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    bad = (c & 0x7F) == 0x7F if fmt == E4M3 else (c & 0x7F) >= 0x7C
    c[bad] &= 0xF0
    return c


def _operands(rng, op, M, N, K, fa, fb):
    if op == 0:
        return _codes(rng, (M, K), fa), _codes(rng, (N, K), fb), (M, N)
    if op == 1:
        return _codes(rng, (M, N), fa), _codes(rng, (N, K), fb), (M, K)
    return _codes(rng, (M, N), fa), _codes(rng, (M, K), fb), (N, K)


_REF = {0: oracle.gemm_fwd, 1: oracle.gemm_dgrad, 2: oracle.gemm_wgrad}

# (op, M, N, K) pairs: the first call's split needs more scratch than the
# second's; the last pair's second product is not split at all.
CASES = [
    ((0, 128, 8192, 8192), (0, 100, 300, 3200)),      # 4 slices of 128 x 8192, then 2 of 100 x 300
    ((1, 2048, 3072, 768), (1, 96, 6400, 80)),        # dX 2048 x 768 in 2 slices, then 96 x 80 in many
    ((2, 6400, 96, 80), (2, 3200, 128, 256)),         # dW 96 x 80, then 128 x 256
    ((0, 16, 48, 6400), (0, 2048, 2048, 1024)),       # one tile in 4 slices, then 256 tiles unsplit
]


@pytest.mark.parametrize("first,second", CASES, ids=[f"op{a[0]}-{a[1]}x{a[2]}x{a[3]}" for a, _ in CASES])
def test_noalloc_matches_the_workspace_entry_point(fl, first, second):
    rng = np.random.default_rng(first[1] * 7 + first[2] + first[3])
    for call, (op, M, N, K) in enumerate((first, second)):
        fa, fb = (E4M3, E4M3) if op == 0 else (E5M2, E4M3)
        a8, b8, shape = _operands(rng, op, M, N, K, fa, fb)
        ba, bb = int(rng.integers(-8, 16)), int(rng.integers(-8, 16))
        A, B, BA, BB = u8_dev(a8), u8_dev(b8), i32_dev(ba), i32_dev(bb)
        nbytes = fl.gemm_workspace_bytes(op, M, N, K)
        assert nbytes <= fl.NOALLOC_SCRATCH_BYTES
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        say("noalloc call", call, "op", op, "MNK", M, N, K, "split bytes", nbytes)
        want = fl.scaled_gemm(op, A, fa, BA, B, fb, BB, workspace=ws)
        out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        got = fl.scaled_gemm_noalloc(op, A, fa, BA, B, fb, BB, out)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (call, op, M, N, K)
        ref, bound = _REF[op](a8, fa, ba, b8, fb, bb)
        check_gemm(got.cpu().numpy(), ref, bound, f"noalloc call {call} op {op} {M}x{N}x{K}")


def test_noalloc_native_arithmetic_matches_the_workspace_entry_point(fl):
    rng = np.random.default_rng(5)
    for (M, N, K) in ((128, 512, 4096), (64, 256, 2048)):
        a8, b8, shape = _operands(rng, 0, M, N, K, E4M3, E4M3)
        A, B, BA, BB = u8_dev(a8), u8_dev(b8), i32_dev(1), i32_dev(2)
        ws = torch.empty(fl.gemm_workspace_bytes(0, M, N, K), dtype=torch.uint8, device="cuda")
        say("noalloc native", M, N, K)
        want = fl.scaled_gemm(0, A, E4M3, BA, B, E4M3, BB, math=fl.MATH_NATIVE_FP8, workspace=ws)
        out = torch.empty(shape, dtype=torch.float32, device="cuda")
        got = fl.scaled_gemm_noalloc(0, A, E4M3, BA, B, E4M3, BB, out, math=fl.MATH_NATIVE_FP8)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (M, N, K)


def test_noalloc_plans_within_its_scratch(fl):
    """A caller's workspace may be planned for two workgroups per CU; the
    no-allocation product takes that plan only where it fits the static
    scratch.  65 x 28672 (224 tiles of 128 x 128, contraction 8192): two
    slices, 14.9 MB, the same plan both ways, the same bits.  192 x 10240
    (160 tiles): three slices, 23.6 MB, past the scratch, so the
    no-allocation product runs unsplit -- the bits of fp8_scaled_gemm; the
    split result within the oracle's bound.  Sampled outputs (the last rows
    and columns among them) against the oracle."""
    rng = np.random.default_rng(11)
    for (M, N, K), same_plan in (((65, 28672, 8192), True), ((192, 10240, 8192), False)):
        a8, b8, shape = _operands(rng, 0, M, N, K, E4M3, E4M3)
        A, B, BA, BB = u8_dev(a8), u8_dev(b8), i32_dev(2), i32_dev(-1)
        nbytes = fl.gemm_workspace_bytes(0, M, N, K)
        assert (nbytes <= fl.NOALLOC_SCRATCH_BYTES) == same_plan, nbytes
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        say("noalloc plan", M, N, K, "workspace plan bytes", nbytes)
        split = fl.scaled_gemm(0, A, E4M3, BA, B, E4M3, BB, workspace=ws)
        plain = fl.scaled_gemm(0, A, E4M3, BA, B, E4M3, BB)
        out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        got = fl.scaled_gemm_noalloc(0, A, E4M3, BA, B, E4M3, BB, out)
        torch.cuda.synchronize()
        want = split if same_plan else plain
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (M, N, K)
        rows = np.concatenate([rng.integers(0, M, 300), M - 1 - np.arange(20)])
        cols = np.concatenate([rng.integers(0, N, 300), N - 1 - np.arange(20)])
        ref, bound = oracle.gemm_fwd_at(a8, E4M3, 2, b8, E4M3, -1, rows, cols)
        for name, res in (("noalloc", got), ("split", split)):
            check_gemm(res.cpu().numpy()[rows, cols], ref, bound, f"{name} {M}x{N}x{K}")
