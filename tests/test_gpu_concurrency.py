"""Concurrent calls: several host threads, each on its own HIP stream, run the
quantisation and the three products at once; every result equals the same
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
    return [x8, bx, ax, w8, bw, aw, g8, bg, ag, y, dx, dw]


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
