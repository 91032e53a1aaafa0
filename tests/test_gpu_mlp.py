"""GPU parity of the chained FP8 MLP: the SwiGLU kernels and every stage of the
forward and backward against the CPU oracle.

Stages are compared one at a time, each fed the GPU's own input to that stage
(its previous stage's output), so that every quantisation decision is taken on
the same values on both sides:
  * amax, bias and FP8 codes: bit-exact;
  * products: |gpu - oracle| <= 1e-5 * 2^-(ba+bb) * sum |a||b| elementwise;
  * SwiGLU (fp32 arithmetic rounded to bf16): within half a bf16 unit in the
    last place of the exact (fp64) value plus the fp32 rounding, i.e.
    |gpu - exact| <= 2^-8 * |exact| * (1 + 2^-10) + 2^-133; the gate gradient
    also allows 2^-20 * |da * u| * (1 + |g|) for the cancellation in
    1 + g * (1 - sigmoid(g)) near its zero (g ~ -1.28).  The amax each kernel
    folds is bit-exact against max |output|.
The end-to-end test compares the autograd Function with the unquantised MLP in
float64 (FP8 rounding error only) and checks that a transposed operand would
fail it.  Method: "Training and inference of large language models using 8-bit
floating point", review page, "Proposed method", bullets 1-5; the SwiGLU
reading: Llama 2's MLP ("Main findings").
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_gemm, f32_dev, need_gpu, say, words_of

pytestmark = pytest.mark.gpu
E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def fl():
    return need_gpu()


def bf16_values(words):
    return (np.asarray(words, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def check_bf16(got_words, exact, what, extra=None, min_same=0.999):
    """Elementwise bf16-rounding tolerance (see the module docstring); on
    random data also nearly every value is the correctly rounded one
    (min_same; None for hand-picked values such as the derivative's zero)."""
    got = bf16_values(got_words).reshape(exact.shape)
    nan_g, nan_e = np.isnan(got), np.isnan(exact)
    assert np.array_equal(nan_g, nan_e), f"{what}: NaN positions differ"
    inf_e = np.isinf(exact)
    assert np.array_equal(got[inf_e], exact[inf_e]), f"{what}: infinities differ"
    m = ~nan_e & ~inf_e
    err = np.abs(got[m] - exact[m])
    tol = 2.0 ** -8 * np.abs(exact[m]) * (1 + 2.0 ** -10) + 2.0 ** -133
    if extra is not None:
        tol = tol + extra[m]
    bad = np.where(err > tol)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {m.sum()} outside; first got {got[m][i]!r} "
                             f"exact {exact[m][i]!r} tol {tol[i]!r}")
    if min_same is None:
        return
    rne = torch.from_numpy(exact[m]).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    same = float(np.mean(got[m] == rne)) if m.any() else 1.0
    assert same >= min_same, f"{what}: only {same:.5f} equal to the rounded exact value"


def amax_bits_of_bf16(words):
    w = np.asarray(words, dtype=np.uint16).reshape(-1)
    return int((w & 0x7FFF).max()) << 16 if w.size else 0


def draw_h(rows, f, seed, scale=3.0):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((rows, 2 * f)) * scale).astype(np.float32)
    da = (rng.standard_normal((rows, f)) * 1e-3).astype(np.float32)
    return h, da


@pytest.mark.parametrize("rows,f", [(1, 1), (3, 5), (7, 64), (33, 130), (129, 1000), (64, 1023), (5, 4097)])
def test_swiglu_forward_and_backward(fl, rows, f):
    h, da = draw_h(rows, f, rows * 1000 + f)
    hd, dad = torch.from_numpy(h).cuda(), torch.from_numpy(da).cuda()
    say("swiglu", rows, f)
    amax_a = torch.empty(1, dtype=torch.float32, device="cuda")
    a = fl.swiglu_fwd(hd, amax=amax_a)
    amax_d = torch.empty(1, dtype=torch.float32, device="cuda")
    dh = fl.swiglu_bwd(hd, dad, amax=amax_d)
    wa, wd = words_of(a), words_of(dh)
    check_bf16(wa, oracle.swiglu_fwd(h), f"fwd {rows}x{f}")
    g, u = h[:, :f].astype(np.float64), h[:, f:].astype(np.float64)
    extra = np.concatenate([2.0 ** -20 * np.abs(da * u) * (1 + np.abs(g)), np.zeros_like(g)], axis=1)
    check_bf16(wd, oracle.swiglu_bwd(h, da), f"bwd {rows}x{f}", extra)
    assert int(words_of(amax_a)[0]) == amax_bits_of_bf16(wa)
    assert int(words_of(amax_d)[0]) == amax_bits_of_bf16(wd)
    # the amax equals fp8_amax over the output
    assert int(words_of(fl.amax(a))[0]) == int(words_of(amax_a)[0])
    # without an amax pointer the outputs are the same
    assert torch.equal(fl.swiglu_fwd(hd).view(torch.int16), a.view(torch.int16))


def test_swiglu_special_values(fl):
    gs = [0.0, -0.0, 1e-40, -1e-40, -87.0, -88.5, -89.0, -95.0, -100.0, -104.0, -110.0, 20.0, 88.0,
          89.0, 100.0, 1e30, -1e30, -1.2784645, 3e38, -3e38, np.inf, -np.inf, np.nan]
    us = [1.0, -2.5, 0.0, 3.0, 1e-30, -4.0]
    g = np.array([x for x in gs for _ in us], dtype=np.float32)
    u = np.array([y for _ in gs for y in us], dtype=np.float32)
    f = g.size
    h = np.concatenate([g, u])[None, :].astype(np.float32)
    da = np.full((1, f), 0.75, dtype=np.float32)
    hd, dad = torch.from_numpy(h).cuda(), torch.from_numpy(da).cuda()
    say("swiglu specials", f)
    a = words_of(fl.swiglu_fwd(hd))
    dh = words_of(fl.swiglu_bwd(hd, dad))
    with np.errstate(all="ignore"):
        ea = oracle.swiglu_fwd(h)
        ed = oracle.swiglu_bwd(h, da)
        gg, uu = g.astype(np.float64)[None, :], u.astype(np.float64)[None, :]
        extra = np.concatenate([np.nan_to_num(2.0 ** -20 * np.abs(0.75 * uu) * (1 + np.abs(gg)), posinf=0.0),
                                np.zeros_like(gg)], axis=1)
    # beyond the bf16 range the rounded value is infinite
    big = 3.3961e38
    with np.errstate(invalid="ignore"):
        ea = np.where(np.isfinite(ea) & (np.abs(ea) >= big), np.sign(ea) * np.inf, ea)
        ed = np.where(np.isfinite(ed) & (np.abs(ed) >= big), np.sign(ed) * np.inf, ed)
    check_bf16(a, ea, "fwd specials", min_same=None)
    check_bf16(dh, ed, "bwd specials", extra, min_same=None)


def test_swiglu_argument_checks_and_empty(fl):
    L = fl.lib
    h = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    a = torch.zeros((4, 4), dtype=torch.bfloat16, device="cuda")
    am = torch.full((1,), 5.0, device="cuda")
    assert L.fp8_swiglu_fwd(h.data_ptr(), -1, 4, a.data_ptr(), None, None) == -2
    assert L.fp8_swiglu_fwd(None, 4, 4, a.data_ptr(), None, None) == -1
    assert L.fp8_swiglu_fwd(h.data_ptr() + 4, 4, 4, a.data_ptr(), None, None) == -5
    assert L.fp8_swiglu_fwd(h.data_ptr(), 4, 4, a.data_ptr(), am.data_ptr() + 2, None) == -5
    assert L.fp8_swiglu_bwd(h.data_ptr(), None, 4, 4, a.data_ptr(), None, None) == -1
    # empty output: only the amax clear runs
    assert L.fp8_swiglu_fwd(None, 0, 4, None, am.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert am.item() == 0.0


def small_mlp(T, d, f, seed, x_dist="normal"):
    m = synth.ChainedMLP(90 + seed, "small", T, d, f, x_dist=x_dist, g_sigma=1e-4)
    return {n: synth.chained_mlp_tensor(m, n) for n in m.ORDER}


def stagewise(fl, t, cfg=None, sample=None):
    """Run mlp_forward / mlp_backward on the GPU and check every stage against
    the oracle on the GPU's own stage inputs.  sample: None for full outputs,
    else the number of sampled outputs per product (and rows for SwiGLU)."""
    from fp8_precision_linear_amd import mlp
    cfg = cfg or mlp.MLPConfig()
    x, w1, w2, g = (t[n].cuda() for n in ("X", "W1", "W2", "G"))
    T, d = x.shape
    f = w2.shape[1]
    say("mlp stagewise", T, d, f, "sample", sample)
    y, s = mlp.mlp_forward(x, w1, w2, cfg)
    dx, dw1, dw2, b = mlp.mlp_backward(s, g, cfg)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    m = cfg.margins

    def quant_ok(src, fmt, margin, codes, bias, what):
        words = words_of(src).reshape(-1)
        a_bits = oracle.amax_bits(words)
        b_ref = oracle.compute_bias(a_bits, fmt, margin)
        assert int(bias.item()) == b_ref, what
        got = codes.cpu().numpy().reshape(-1)
        assert np.array_equal(got, oracle.scale_cast(words, b_ref, fmt)), what
        return b_ref

    bx = quant_ok(t["X"], E4M3, m["x"], s["x8"], s["bx"], "x")
    bw1 = quant_ok(t["W1"], E4M3, m["w1"], s["w1_8"], s["bw1"], "w1")
    bw2 = quant_ok(t["W2"], E4M3, m["w2"], s["w2_8"], s["bw2"], "w2")
    x8, w1_8, w2_8 = s["x8"].cpu().numpy(), s["w1_8"].cpu().numpy(), s["w2_8"].cpu().numpy()

    def prod(kind, got, a8, fa, ba, b8, fb, bb, what):
        full = {"fwd": oracle.gemm_fwd, "dgrad": oracle.gemm_dgrad, "wgrad": oracle.gemm_wgrad}[kind]
        at = {"fwd": oracle.gemm_fwd_at, "dgrad": oracle.gemm_dgrad_at, "wgrad": oracle.gemm_wgrad_at}[kind]
        got = got.cpu().numpy()
        if sample is None:
            ref, bound = full(a8, fa, ba, b8, fb, bb)
            check_gemm(got, ref, bound, what)
        else:
            rows = rng.integers(0, got.shape[0], sample)
            cols = rng.integers(0, got.shape[1], sample)
            ref, bound = at(a8, fa, ba, b8, fb, bb, rows, cols)
            check_gemm(got[rows, cols], ref, bound, what)

    prod("fwd", s["h"], x8, E4M3, bx, w1_8, E4M3, bw1, "h = x8 . w1_8^T")
    # SwiGLU on the GPU's h (all rows, or sampled rows)
    h = s["h"]
    ridx = np.arange(T) if sample is None else np.sort(rng.choice(T, min(16, T), replace=False))
    h_rows = h[torch.from_numpy(ridx).cuda()].cpu().numpy()
    a_words = words_of(s["a"])
    check_bf16(a_words[ridx], oracle.swiglu_fwd(h_rows), "a = silu(g) * u")
    assert int(words_of(s["a_amax"])[0]) == amax_bits_of_bf16(a_words), "amax(a)"
    ba = quant_ok(s["a"], E4M3, m["a"], s["a8"], s["ba"], "a")
    a8 = s["a8"].cpu().numpy()
    prod("fwd", y, a8, E4M3, ba, w2_8, E4M3, bw2, "y = a8 . w2_8^T")
    # backward
    bdy = quant_ok(t["G"], E5M2, m["dy"], b["dy8"], b["bdy"], "dy")
    dy8 = b["dy8"].cpu().numpy()
    prod("dgrad", b["da"], dy8, E5M2, bdy, w2_8, E4M3, bw2, "da = dy8 . w2_8")
    prod("wgrad", dw2, dy8, E5M2, bdy, a8, E4M3, ba, "dw2 = dy8^T . a8")
    da_rows = b["da"][torch.from_numpy(ridx).cuda()].cpu().numpy()
    dh_words = words_of(b["dh"])
    gg, uu = h_rows[:, :f].astype(np.float64), h_rows[:, f:].astype(np.float64)
    extra = np.concatenate([2.0 ** -20 * np.abs(da_rows * uu) * (1 + np.abs(gg)), np.zeros_like(gg)], axis=1)
    check_bf16(dh_words[ridx], oracle.swiglu_bwd(h_rows, da_rows), "dh", extra)
    assert int(words_of(b["dh_amax"])[0]) == amax_bits_of_bf16(dh_words), "amax(dh)"
    bdh = quant_ok(b["dh"], E5M2, m["dh"], b["dh8"], b["bdh"], "dh")
    dh8 = b["dh8"].cpu().numpy()
    prod("dgrad", dx, dh8, E5M2, bdh, w1_8, E4M3, bw1, "dx = dh8 . w1_8")
    prod("wgrad", dw1, dh8, E5M2, bdh, x8, E4M3, bx, "dw1 = dh8^T . x8")
    return y, dx, dw1, dw2


@pytest.mark.parametrize("T,d,f", [(96, 128, 80), (70, 96, 70), (130, 64, 200)])
def test_mlp_every_stage_small(fl, T, d, f):
    stagewise(fl, small_mlp(T, d, f, T % 7), sample=None)


def test_mlp_every_stage_with_margins(fl):
    from fp8_precision_linear_amd import mlp
    cfg = mlp.MLPConfig(margins={"x": 1, "w1": 0, "a": 2, "w2": -1, "dy": 3, "dh": 1})
    stagewise(fl, small_mlp(64, 128, 96, 3, x_dist="t3_outliers"), cfg=cfg)


def test_mlp_llama7b_shapes_sampled(fl):
    """The bench's chained-MLP workload at its full size, sampled outputs."""
    m = synth.CHAINED_MLPS[6]
    t = {n: synth.chained_mlp_tensor(m, n) for n in m.ORDER}
    stagewise(fl, t, sample=4096)


def test_mlp_small_batch_split_products(fl):
    """The Llama-2-7B MLP with 32 tokens: the down projection, its data
    gradient and the input's data gradient have outputs of 32 x 4096 or
    32 x 11008 (a few tiles), so they run split along the contraction
    (fp8_scaled_gemm_ws); every stage against the oracle, products in full."""
    T, d, f = 32, 4096, 11008
    assert fl.gemm_workspace_bytes(fl.OP_FWD, T, d, f) > 0
    assert fl.gemm_workspace_bytes(fl.OP_DGRAD, T, d, f) > 0
    assert fl.gemm_workspace_bytes(fl.OP_DGRAD, T, 2 * f, d) > 0
    stagewise(fl, small_mlp(T, d, f, 5), sample=None)


def reference_fp64(t):
    x = t["X"].double().requires_grad_()
    w1 = t["W1"].double().requires_grad_()
    w2 = t["W2"].double().requires_grad_()
    f = w2.shape[1]
    h = x @ w1.T
    y = (torch.nn.functional.silu(h[:, :f]) * h[:, f:]) @ w2.T
    y.backward(t["G"].double())
    return y.detach(), x.grad, w1.grad, w2.grad


def rel(a, b):
    return float(torch.linalg.norm(a.double().cpu() - b) / torch.linalg.norm(b))


def test_autograd_function_end_to_end(fl):
    from fp8_precision_linear_amd import mlp
    t = small_mlp(128, 256, 192, 5)
    x = t["X"].cuda().requires_grad_()
    w1 = t["W1"].cuda().requires_grad_()
    w2 = t["W2"].cuda().requires_grad_()
    log = mlp.BiasLog()
    cfg = mlp.MLPConfig(log=log)
    say("mlp autograd")
    y = mlp.FP8MLPFunction.apply(x, w1, w2, cfg)
    y.backward(t["G"].cuda())
    torch.cuda.synchronize()
    ry, rdx, rdw1, rdw2 = reference_fp64(t)
    errs = {"y": rel(y.detach(), ry), "dx": rel(x.grad.float(), rdx), "dw1": rel(w1.grad, rdw1),
            "dw2": rel(w2.grad, rdw2)}
    print("relative errors vs unquantised fp64", errs)
    # FP8 rounding alone (E4M3 forward, E5M2 gradients): a few per cent
    for k, e in errs.items():
        assert e < 0.2, (k, e)
    # a transposed or swapped operand is far outside that
    assert rel(y.detach(), ry.flip(1)) > 0.8
    # the Function is exactly mlp_forward / mlp_backward
    y2, s = mlp.mlp_forward(t["X"].cuda(), t["W1"].cuda(), t["W2"].cuda())
    dx2, dw1_2, dw2_2, _ = mlp.mlp_backward(s, t["G"].cuda())
    assert torch.equal(y.detach(), y2) and torch.equal(w1.grad, dw1_2) and torch.equal(w2.grad, dw2_2)
    assert torch.equal(x.grad, dx2.to(x.dtype))
    hist = log.history()
    assert all(len(hist[n]) == 1 for n in mlp.TENSORS)
    assert hist["x"][0] == int(s["bx"].item()) and hist["a"][0] == int(s["ba"].item())


def test_bias_log_over_training_steps(fl):
    """A few Adam steps on a synthetic regression: the loss falls and every
    logged bias is the one the oracle computes from that step's tensor."""
    from fp8_precision_linear_amd import mlp
    t = small_mlp(256, 128, 128, 6)
    torch.manual_seed(0)
    teacher_w1 = (torch.randn(256, 128) * 0.1).cuda()
    x = t["X"].cuda()
    with torch.no_grad():
        hh = x.float() @ teacher_w1.T
        target = (torch.nn.functional.silu(hh[:, :128]) * hh[:, 128:]) @ (torch.randn(128, 128) * 0.1).cuda().T
    model = mlp.FP8SwiGLUMLP(128, 128, device="cuda")
    log = mlp.BiasLog()
    model.cfg.log = log
    opt = torch.optim.Adam(model.parameters(), lr=1e-2)
    losses, w1_words = [], []
    for step in range(8):
        say("train step", step)
        w1_words.append(words_of(model.w1.detach()).copy())
        y = model(x)
        loss = ((y - target) ** 2).mean()
        opt.zero_grad()
        loss.backward()
        opt.step()
        losses.append(loss.item())
    print("losses", losses)
    assert losses[-1] < 0.8 * losses[0]       # unquantised float64: 0.84 -> 0.46
    hist = log.history()
    assert all(len(hist[n]) == 8 for n in mlp.TENSORS)
    for step in range(8):
        assert hist["w1"][step] == oracle.compute_bias(oracle.amax_bits(w1_words[step]), E4M3, 0)
    print("bias history", hist)


def test_mlp_step_replays_in_a_hip_graph(fl):
    """The chained MLP's forward + backward captured once into a HIP graph
    (torch.cuda.CUDAGraph) and replayed: every replay, with eager work and
    synchronisations between replays and the inputs changed in place, equals
    the eager step bit for bit (the library's clears are kernels, not memsets,
    and nothing in the step synchronises with the host)."""
    from fp8_precision_linear_amd import mlp
    t = small_mlp(256, 256, 192, 8)
    x = t["X"].cuda()
    w1 = t["W1"].cuda().requires_grad_()
    w2 = t["W2"].cuda().requires_grad_()
    g = t["G"].cuda()
    cfg = mlp.MLPConfig()

    def step():
        w1.grad = None
        w2.grad = None
        y = mlp.FP8MLPFunction.apply(x, w1, w2, cfg)
        y.backward(g)
        return y

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    say("mlp graph capture")
    with torch.cuda.graph(graph, stream=side):
        y_g = step()
    dw1_g, dw2_g = w1.grad, w2.grad
    rng = np.random.default_rng(9)
    for r in range(4):
        # new inputs, in place (the graph reads these buffers)
        with torch.no_grad():
            x.copy_(synth.to_bf16((rng.standard_normal(tuple(x.shape)) * (1 + r)).astype(np.float32)).cuda())
            w1.mul_(0.9)
            g.mul_(2.0)
        say("mlp graph replay", r)
        graph.replay()
        torch.cuda.synchronize()
        got = (y_g.clone(), dw1_g.clone(), dw2_g.clone())
        # eager step on the same inputs, with other eager work in between (on
        # the warm-up stream, where the weights' gradient nodes were made)
        _ = torch.randn(1000, device="cuda").sum()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            y_e = step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], y_e.detach()), r
        assert torch.equal(got[1], w1.grad) and torch.equal(got[2], w2.grad), r
