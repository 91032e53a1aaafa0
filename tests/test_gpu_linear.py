"""GPU parity of the FP8-AMAX linear layer (autograd Function and module)
against the CPU oracle, in both scaling modes.

"Training and inference of large language models using 8-bit floating point",
review page, "Proposed method", bullets 1-5: the input and the weight (E4M3)
and the output gradient (E5M2) quantised per tensor, the three products in
FP8 and unscaled.  Codes and biases are bit-exact; products within
1e-5 * 2^-(ba+bb) * sum |a||b|, each stage fed the GPU's own inputs.  Delayed
scaling: step t's bias is the oracle's bias of step t-1's tensor.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_gemm, need_gpu, say, words_of

pytestmark = pytest.mark.gpu
E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def fl():
    return need_gpu()


def tensors(shape_x, n_out, seed, x_scale=1.0, g_scale=1e-4):
    rng = np.random.default_rng(seed)
    x = synth.to_bf16((rng.standard_normal(shape_x) * x_scale).astype(np.float32))
    w = torch.from_numpy((rng.standard_normal((n_out, shape_x[-1])) * 0.02).astype(np.float32))
    g = torch.from_numpy((rng.standard_normal(shape_x[:-1] + (n_out,)) * g_scale).astype(np.float32))
    return x, w, g


def test_linear_current_scaling_every_stage(fl):
    from fp8_precision_linear_amd import linear, mlp
    x, w, g = tensors((3, 70, 200), 136, 1)            # 210 tokens, K 200, N 136 (ragged)
    log = mlp.BiasLog()
    lin = linear.FP8Linear(200, 136, log=log, device="cuda")
    with torch.no_grad():
        lin.weight.copy_(w)
    xd = x.cuda().requires_grad_()
    say("fp8 linear, current scaling")
    y = lin(xd)
    y.backward(g.cuda())
    torch.cuda.synchronize()
    assert y.shape == (3, 70, 136) and xd.grad.shape == x.shape and lin.weight.grad.shape == w.shape
    xw, ww, gw = synth.bf16_words(x).reshape(210, 200), w.numpy().view(np.uint32), g.numpy().reshape(210, 136).view(np.uint32)
    _, bx, x8 = oracle.quantize(xw, E4M3)
    _, bw, w8 = oracle.quantize(ww, E4M3)
    _, bdy, dy8 = oracle.quantize(gw, E5M2)
    hist = log.history()
    assert hist == {"x": [bx], "w": [bw], "dy": [bdy]}
    ref, bound = oracle.gemm_fwd(x8, E4M3, bx, w8, E4M3, bw)
    check_gemm(y.detach().reshape(210, 136).cpu().numpy(), ref, bound, "linear fwd")
    ref, bound = oracle.gemm_wgrad(dy8, E5M2, bdy, x8, E4M3, bx)
    check_gemm(lin.weight.grad.cpu().numpy(), ref, bound, "linear wgrad")
    ref, bound = oracle.gemm_dgrad(dy8, E5M2, bdy, w8, E4M3, bw)
    # dx comes back in x's dtype (bf16): compare the fp32 product before that
    # rounding through the functional path, and the bf16 result within half a bf16 ulp
    dx32 = fl.scaled_gemm(fl.OP_DGRAD, torch.from_numpy(dy8).cuda(), E5M2, torch.tensor([bdy], dtype=torch.int32, device="cuda"),
                          torch.from_numpy(w8).cuda(), E4M3, torch.tensor([bw], dtype=torch.int32, device="cuda"))
    check_gemm(dx32.cpu().numpy(), ref, bound, "linear dgrad")
    assert torch.equal(xd.grad.reshape(210, 200), dx32.to(torch.bfloat16))


def test_linear_delayed_scaling_uses_the_previous_steps_amax(fl):
    from fp8_precision_linear_amd import linear, mlp
    log = mlp.BiasLog()
    lin = linear.FP8Linear(256, 128, mode="delayed", log=log, device="cuda")
    scales = [1.0, 8.0, 0.5, 0.5, 30.0]
    prev = {}
    for t, sc in enumerate(scales):
        x, _, g = tensors((96, 256), 128, 10 + t, x_scale=sc, g_scale=1e-4 * sc)
        w_words = words_of(lin.weight.detach()).copy()
        xd = x.cuda()
        say("fp8 linear, delayed scaling, step", t)
        lin.weight.grad = None
        y = lin(xd)
        y.backward(g.cuda())
        torch.cuda.synchronize()
        cur = {"x": synth.bf16_words(x), "w": w_words, "dy": g.numpy().view(np.uint32)}
        # the bias of each role: the current tensor's at step 0, else the previous step's
        want = {r: oracle.compute_bias(oracle.amax_bits(prev[r] if t else cur[r]), linear.FORMATS[r], 0)
                for r in linear.ROLES}
        hist = log.history()
        got = {r: hist[r][t] for r in linear.ROLES}
        assert got == want, (t, got, want)
        # the forward product from the codes the oracle makes with those biases
        x8 = oracle.scale_cast(cur["x"], want["x"], E4M3)
        w8 = oracle.scale_cast(cur["w"], want["w"], E4M3)
        ref, bound = oracle.gemm_fwd(x8, E4M3, want["x"], w8, E4M3, want["w"])
        check_gemm(y.detach().cpu().numpy(), ref, bound, f"delayed fwd step {t}")
        dy8 = oracle.scale_cast(cur["dy"], want["dy"], E5M2)
        ref, bound = oracle.gemm_wgrad(dy8, E5M2, want["dy"], x8, E4M3, want["x"])
        check_gemm(lin.weight.grad.cpu().numpy(), ref, bound, f"delayed wgrad step {t}")
        # the state holds this step's amax for the next one
        for r in linear.ROLES:
            assert int(words_of(lin.state.amax[r])[0]) == oracle.amax_bits(cur[r]), (t, r)
        prev = cur
        with torch.no_grad():
            lin.weight.mul_(1.5)


def test_linear_fused_weight_gradient_accumulation(fl):
    """fuse_wgrad_accumulation: three micro-batches' weight gradients summed
    into weight.grad by fp8_scaled_gemm_accumulate (the first pass, with
    weight.grad cleared, writes it).  After micro-batch t, weight.grad
    against the oracle's sum of the t + 1 weight-gradient products (float64,
    from the oracle's codes): within their bounds plus one fp32 rounding per
    addition; the same holds for an unfused layer (autograd adding fp32
    gradients), and dx is the unfused layer's bit for bit."""
    from fp8_precision_linear_amd import linear
    fused = linear.FP8Linear(200, 136, device="cuda", fuse_wgrad_accumulation=True)
    plain = linear.FP8Linear(200, 136, device="cuda")
    _, w, _ = tensors((210, 200), 136, 40)
    with torch.no_grad():
        fused.weight.copy_(w)
        plain.weight.copy_(w)
    _, bw, w8 = oracle.quantize(w.numpy().view(np.uint32), E4M3)
    ref = np.zeros((136, 200))
    bound = np.zeros((136, 200))
    rounding = np.zeros((136, 200))
    for t in range(3):
        x, _, g = tensors((210, 200), 136, 41 + t, x_scale=1.0 + t, g_scale=1e-4 * (3 - t))
        _, bx, x8 = oracle.quantize(synth.bf16_words(x).reshape(210, 200), E4M3)
        _, bdy, dy8 = oracle.quantize(g.numpy().view(np.uint32), E5M2)
        y_ref, y_bound = oracle.gemm_wgrad(dy8, E5M2, bdy, x8, E4M3, bx)
        ref, bound = ref + y_ref, bound + y_bound
        if t:
            rounding += 2.0 ** -24 * np.abs(ref) * (1 + 2.0 ** -20)
        say("fp8 linear, fused weight-gradient accumulation, micro-batch", t)
        grads = {}
        for name, lin in (("fused", fused), ("plain", plain)):
            xd = x.cuda().requires_grad_()
            lin(xd).backward(g.cuda())
            grads[name] = xd.grad
        torch.cuda.synchronize()
        assert torch.equal(grads["fused"], grads["plain"])
        for name, lin in (("fused", fused), ("plain", plain)):
            check_gemm(lin.weight.grad.cpu().numpy(), ref, bound, f"{name} accumulated wgrad, micro-batch {t}",
                       extra=rounding)
    with pytest.raises(ValueError):
        linear.FP8Linear(8, 8, device="cuda", dtype=torch.bfloat16, fuse_wgrad_accumulation=True)


def test_linear_end_to_end_against_unquantised_fp64(fl):
    from fp8_precision_linear_amd import linear
    x, w, g = tensors((512, 384), 256, 3)
    lin = linear.FP8Linear(384, 256, device="cuda")
    with torch.no_grad():
        lin.weight.copy_(w)
    xd = x.cuda().float().requires_grad_()
    y = lin(xd)
    y.backward(g.cuda())
    xr = x.double().requires_grad_()
    wr = w.double().requires_grad_()
    yr = xr @ wr.T
    yr.backward(g.double())
    rel = lambda a, b: float(torch.linalg.norm(a.double().cpu() - b) / torch.linalg.norm(b))
    errs = (rel(y.detach(), yr.detach()), rel(xd.grad, xr.grad), rel(lin.weight.grad, wr.grad))
    print("relative errors (y, dx, dw)", errs)
    assert all(e < 0.1 for e in errs), errs
    assert rel(y.detach(), yr.detach().T.contiguous().T.flip(0)) > 0.8


def test_linear_frozen_weight_for_inference(fl):
    """freeze_weight(): the weight is quantised once; later calls reuse its
    codes (one logged weight bias over several calls, outputs identical to an
    unfrozen layer's on the same weight), even after the weight changes."""
    from fp8_precision_linear_amd import linear, mlp
    x, w, _ = tensors((128, 256), 192, 21)
    log = mlp.BiasLog()
    lin = linear.FP8Linear(256, 192, log=log, device="cuda")
    ref = linear.FP8Linear(256, 192, device="cuda")
    with torch.no_grad():
        lin.weight.copy_(w)
        ref.weight.copy_(w)
    lin.freeze_weight()
    xd = x.cuda()
    with torch.no_grad():
        y_ref = ref(xd)
        outs = [lin(xd) for _ in range(3)]
        lin.weight.mul_(4.0)                 # ignored while frozen
        outs.append(lin(xd))
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, y_ref)
    hist = log.history()
    assert len(hist["w"]) == 1 and len(hist["x"]) == 4
    lin.unfreeze_weight()
    with torch.no_grad():
        assert not torch.equal(lin(xd), y_ref)


@pytest.mark.parametrize("tokens", [1, 32, 100])
def test_linear_small_batch_forward_product(fl, tokens):
    """A few tokens through a 4096 -> 1024 layer: the forward output has 8
    tiles of 128 x 128, so the layer hands its product a workspace
    (fp8_scaled_gemm_ws).  32 tokens: the row kernel takes the product (the
    workspace goes unused); 100 tokens: it runs split along the
    contraction; 1 token: the row kernel as a decoding step would run it.
    Every product against the oracle."""
    from fp8_precision_linear_amd import linear
    x, w, g = tensors((tokens, 4096), 1024, 2)
    assert fl.gemm_workspace_bytes(fl.OP_FWD, tokens, 1024, 4096) > 0
    lin = linear.FP8Linear(4096, 1024, device="cuda")
    with torch.no_grad():
        lin.weight.copy_(w)
    xd = x.cuda().requires_grad_()
    say("fp8 linear, small batch", tokens, "tokens")
    y = lin(xd)
    y.backward(g.cuda())
    torch.cuda.synchronize()
    xw, ww, gw = synth.bf16_words(x), w.numpy().view(np.uint32), g.numpy().view(np.uint32)
    _, bx, x8 = oracle.quantize(xw, E4M3)
    _, bw, w8 = oracle.quantize(ww, E4M3)
    _, bdy, dy8 = oracle.quantize(gw, E5M2)
    ref, bound = oracle.gemm_fwd(x8, E4M3, bx, w8, E4M3, bw)
    check_gemm(y.detach().cpu().numpy(), ref, bound, f"small-batch linear fwd ({tokens} tokens)")
    ref, bound = oracle.gemm_wgrad(dy8, E5M2, bdy, x8, E4M3, bx)
    check_gemm(lin.weight.grad.cpu().numpy(), ref, bound, "small-batch linear wgrad")
    ref, bound = oracle.gemm_dgrad(dy8, E5M2, bdy, w8, E4M3, bw)
    # dx in x's dtype (bf16): within the bound plus half a bf16 ulp of the result
    dx = xd.grad.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(dx - ref) <= 1e-5 * bound + np.abs(ref) * 2.0 ** -8), "small-batch linear dgrad"
