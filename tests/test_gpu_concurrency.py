"""Concurrent calls: several host threads, each on its own HIP stream, run the
quantisation (current and delayed scaling) and the three products at once; every result equals the same
calls run one at a time (the library keeps no state between calls beyond a
per-device architecture flag, and ctypes releases the GIL during a call)."""
import threading

import numpy as np
import pytest
import torch

import synth
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fl():
    return need_gpu()


def work(fl, x, w, g, stream):
    with torch.cuda.stream(stream):
        x8, bx, ax = fl.quantize(x, fl.E4M3, 0, stream=stream)
        w8, bw, aw = fl.quantize(w, fl.E4M3, 1, stream=stream)
        g8, bg, ag = fl.quantize(g, fl.E5M2, 0, stream=stream)
        y = fl.scaled_gemm(fl.OP_FWD, x8, fl.E4M3, bx, w8, fl.E4M3, bw, stream=stream)
        dx = fl.scaled_gemm(fl.OP_DGRAD, g8, fl.E5M2, bg, w8, fl.E4M3, bw, stream=stream)
        dw = fl.scaled_gemm(fl.OP_WGRAD, g8, fl.E5M2, bg, x8, fl.E4M3, bx, stream=stream)
        # delayed scaling: the cast that leaves its block maxima in its own codes
        prev = ax.clone()
        xd8, bxd = fl.quantize_delayed(x, fl.E4M3, prev, 0, stream=stream)
        gam = torch.empty(1, dtype=torch.float32, device=g.device)
        gd8 = fl.scale_cast(g, bg, fl.E5M2, stream=stream, amax=gam)
    return [x8, bx, ax, w8, bw, aw, g8, bg, ag, y, dx, dw, xd8, bxd, prev, gd8, gam]


def test_threads_on_separate_streams(fl):
    nthreads, reps = 4, 6
    inputs = []
    for t in range(nthreads):
        x = synth.draw_bf16(500 + t, (1024, 512), "normal", 1.0 + t).cuda()
        w = synth.draw_bf16(600 + t, (768, 512), "normal", 0.02).cuda()
        g = synth.draw_bf16(700 + t, (1024, 768), "normal", 1e-4).cuda()
        inputs.append((x, w, g))
    say("concurrency: serial references")
    ref = [work(fl, *inputs[t], torch.cuda.current_stream()) for t in range(nthreads)]
    torch.cuda.synchronize()
    results = [[None] * reps for _ in range(nthreads)]
    errors = []

    def run(t):
        try:
            s = torch.cuda.Stream()
            for r in range(reps):
                results[t][r] = work(fl, *inputs[t], s)
            s.synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    say("concurrency: threads")
    threads = [threading.Thread(target=run, args=(t,)) for t in range(nthreads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(nthreads):
        for r in range(reps):
            for a, b in zip(results[t][r], ref[t]):
                assert torch.equal(a, b), (t, r)


def test_side_stream_without_a_stream_context(fl):
    """A call given another stream than torch's current one, outside any
    stream context: its outputs and a split product's workspace are allocated
    on that stream, so memory the current stream allocates and fills right
    after the call cannot be the blocks the call is still writing.  Results
    equal the same calls on the current stream."""
    import oracle
    from gpu_util import check_gemm

    x = synth.draw_bf16(810, (128, 8192), "normal", 1.0).cuda()
    w = synth.draw_bf16(811, (1024, 8192), "normal", 0.02).cuda()
    x8, bx, _ = fl.quantize(x, fl.E4M3, 0)
    w8, bw, _ = fl.quantize(w, fl.E4M3, 0)
    assert fl.gemm_workspace_bytes(fl.OP_FWD, 128, 1024, 8192) > 0      # split: a workspace
    want = fl.scaled_gemm_auto(fl.OP_FWD, x8, fl.E4M3, bx, w8, fl.E4M3, bw)
    q_want = fl.quantize(x, fl.E4M3, 0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        say("side stream", rep)
        y = fl.scaled_gemm_auto(fl.OP_FWD, x8, fl.E4M3, bx, w8, fl.E4M3, bw, stream=side)
        codes, bias, amax = fl.quantize(x, fl.E4M3, 0, stream=side)
        # the current stream allocates and overwrites fresh memory meanwhile
        junk = [torch.full((1 << 22,), float(rep), device="cuda") for _ in range(8)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), want.view(torch.int32)), rep
        assert torch.equal(codes, q_want[0]) and torch.equal(bias, q_want[1]), rep
        del junk, y, codes, bias, amax
    ref, bound = oracle.gemm_fwd(x8.cpu().numpy(), 0, int(bx.item()), w8.cpu().numpy(), 0, int(bw.item()))
    check_gemm(want.cpu().numpy(), ref, bound, "side-stream product")
