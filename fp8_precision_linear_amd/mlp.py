"""Chained FP8 MLP: Llama 2's gated MLP with every product an FP8-AMAX scaled
GEMM, as a PyTorch autograd Function.

"Training and inference of large language models using 8-bit floating point",
review page, "Proposed method": each weight, activation and gradient tensor is
scaled by 2^bias from its own amax (bullets 1-2), cast to E4M3 (weights,
activations) or E5M2 (gradients) (bullet 4), multiplied in FP8 and unscaled
(bullet 3), in training (bullet 5).  The pages train Llama 2 models ("Main
findings"); the activation between that model's MLP products, SwiGLU, is not
spelled out there and is taken as a = silu(g) * u.

Forward (x [T, d], w1 = [W_gate; W_up] [2F, d], w2 = W_down [d, F]):
    x8  = cast_E4(x),  w1_8 = cast_E4(w1),  w2_8 = cast_E4(w2)
                                     amax -> bias -> cast each, the three in one call
    h   = x8 . w1_8^T                [T, 2F] fp32  (gate columns, then up)
    a   = silu(g) * u                [T, F]  bf16, amax folded in the kernel
    a8  = cast_E4(a)
    y   = a8 . w2_8^T                [T, d]  fp32
Backward (dy [T, d]):
    dy8 = cast_E5(dy)
    da  = dy8 . w2_8                 [T, F]  fp32     dw2 = dy8^T . a8  [d, F]
    dh  = [da*u*silu'(g) | da*silu(g)]  [T, 2F] bf16, amax folded in the kernel
    dh8 = cast_E5(dh)
    dx  = dh8 . w1_8                 [T, d]  fp32     dw1 = dh8^T . x8  [2F, d]

The fused gate-up weight is one tensor with one scale, and so is its gradient
[dG | dU].  Every step runs in libfp8lin's kernels on the current stream with
no host synchronisation; this module only allocates outputs (and the
workspace of a product split along the contraction, for small batches) and
orders the calls.  Gradients come back in fp32 (autograd converts dx to x's dtype).
"""
from contextlib import contextmanager
from dataclasses import dataclass, field

import torch

from . import (E4M3, E5M2, MATH_EXACT, OP_DGRAD, OP_FWD, OP_WGRAD, compute_bias, quantize,
               quantize_multi, scale_cast, scaled_gemm_auto, swiglu_bwd, swiglu_fwd)

# The quantised tensors of one forward + backward, in log order.
TENSORS = ("x", "w1", "a", "w2", "dy", "dh")
FORMATS = {"x": E4M3, "w1": E4M3, "a": E4M3, "w2": E4M3, "dy": E5M2, "dh": E5M2}


class BiasLog:
    """Per-tensor scaling biases of every forward and backward, kept as device
    tensors (no synchronisation) until `history` reads them: the per-tensor
    scale record the pages plot over training."""

    def __init__(self):
        self._events = []   # (tensor name, int32[1] device tensor), in call order

    def record(self, name, bias):
        self._events.append((name, bias))

    def history(self):
        """{tensor name: [bias per call]}, names in order of first use (one
        host read of all of them)."""
        out = {}
        for n, _ in self._events:
            out.setdefault(n, [])
        if self._events:
            vals = torch.cat([b for _, b in self._events]).cpu().tolist()
            for (n, _), v in zip(self._events, vals):
                out[n].append(int(v))
        return out


@dataclass
class MLPConfig:
    """Margins per quantised tensor (compute_bias's margin), the product
    arithmetic, an optional bias log, and an optional list that receives
    (kind, name, start event, end event) around every group of launches
    (kind: "quant", "gemm" or "swiglu"), for per-kernel timing."""
    margins: dict = field(default_factory=lambda: {n: 0 for n in TENSORS})
    math: int = MATH_EXACT
    log: BiasLog = None
    events: list = None


@contextmanager
def _span(cfg, kind, name):
    if cfg.events is None:
        yield
        return
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    yield
    e1.record()
    cfg.events.append((kind, name, e0, e1))


def _shapes(x, w1, w2):
    if x.dim() != 2 or w1.dim() != 2 or w2.dim() != 2:
        raise ValueError("x [T, d], w1 [2F, d] and w2 [d, F] must be 2-D")
    T, d = x.shape
    f2, d1 = w1.shape
    d2, f = w2.shape
    if d1 != d or d2 != d or f2 != 2 * f:
        raise ValueError(f"shapes do not chain: x {tuple(x.shape)}, w1 {tuple(w1.shape)}, "
                         f"w2 {tuple(w2.shape)}")
    return T, d, f


def mlp_forward(x, w1, w2, cfg=None):
    """y and the tensors the backward needs (a dict, also holding the
    intermediates h and a and every code tensor and bias)."""
    cfg = cfg or MLPConfig()
    _shapes(x, w1, w2)
    m = cfg.margins
    a_amax = torch.empty(1, dtype=torch.float32, device=x.device)
    # the three inputs known at the start in one call (three launches for all)
    with _span(cfg, "quant", "x+w1+w2"):
        (x8, bx, _), (w1_8, bw1, _), (w2_8, bw2, _) = quantize_multi(
            [x, w1, w2], E4M3, [m["x"], m["w1"], m["w2"]])
    with _span(cfg, "gemm", "fwd h"):
        h = scaled_gemm_auto(OP_FWD, x8, E4M3, bx, w1_8, E4M3, bw1, math=cfg.math)
    with _span(cfg, "swiglu", "fwd"):
        a = swiglu_fwd(h, amax=a_amax)
    with _span(cfg, "quant", "a"):
        ba = compute_bias(a_amax, E4M3, m["a"])
        a8 = scale_cast(a, ba, E4M3)
    with _span(cfg, "gemm", "fwd y"):
        y = scaled_gemm_auto(OP_FWD, a8, E4M3, ba, w2_8, E4M3, bw2, math=cfg.math)
    if cfg.log is not None:
        for n, b in (("x", bx), ("w1", bw1), ("a", ba), ("w2", bw2)):
            cfg.log.record(n, b)
    return y, {"x8": x8, "bx": bx, "w1_8": w1_8, "bw1": bw1, "h": h, "a": a, "a_amax": a_amax,
               "a8": a8, "ba": ba, "w2_8": w2_8, "bw2": bw2}


def mlp_backward(saved, dy, cfg=None):
    """(dx, dw1, dw2, intermediates) from the forward's saved tensors."""
    cfg = cfg or MLPConfig()
    m = cfg.margins
    dy = dy.contiguous()
    dh_amax = torch.empty(1, dtype=torch.float32, device=dy.device)
    with _span(cfg, "quant", "dy"):
        dy8, bdy, _ = quantize(dy, E5M2, m["dy"])
    with _span(cfg, "gemm", "dgrad da"):
        da = scaled_gemm_auto(OP_DGRAD, dy8, E5M2, bdy, saved["w2_8"], E4M3, saved["bw2"], math=cfg.math)
    with _span(cfg, "gemm", "wgrad dw2"):
        dw2 = scaled_gemm_auto(OP_WGRAD, dy8, E5M2, bdy, saved["a8"], E4M3, saved["ba"], math=cfg.math)
    with _span(cfg, "swiglu", "bwd"):
        dh = swiglu_bwd(saved["h"], da, amax=dh_amax)
    with _span(cfg, "quant", "dh"):
        bdh = compute_bias(dh_amax, E5M2, m["dh"])
        dh8 = scale_cast(dh, bdh, E5M2)
    with _span(cfg, "gemm", "dgrad dx"):
        dx = scaled_gemm_auto(OP_DGRAD, dh8, E5M2, bdh, saved["w1_8"], E4M3, saved["bw1"], math=cfg.math)
    with _span(cfg, "gemm", "wgrad dw1"):
        dw1 = scaled_gemm_auto(OP_WGRAD, dh8, E5M2, bdh, saved["x8"], E4M3, saved["bx"], math=cfg.math)
    if cfg.log is not None:
        cfg.log.record("dy", bdy)
        cfg.log.record("dh", bdh)
    return dx, dw1, dw2, {"dy8": dy8, "bdy": bdy, "da": da, "dh": dh, "dh_amax": dh_amax,
                          "dh8": dh8, "bdh": bdh}


class FP8MLPFunction(torch.autograd.Function):
    """y = FP8 MLP(x; w1, w2); gradients for x, w1 and w2."""

    @staticmethod
    def forward(ctx, x, w1, w2, cfg):
        y, saved = mlp_forward(x.contiguous(), w1.contiguous(), w2.contiguous(), cfg)
        ctx.saved = saved
        ctx.cfg = cfg
        return y

    @staticmethod
    def backward(ctx, dy):
        dx, dw1, dw2, _ = mlp_backward(ctx.saved, dy, ctx.cfg)
        ctx.saved = None
        return dx, dw1, dw2, None


class FP8SwiGLUMLP(torch.nn.Module):
    """The gated MLP with FP8-AMAX products: parameters w1 = [W_gate; W_up]
    [2F, d] and w2 = W_down [d, F] (fp32 master weights by default)."""

    def __init__(self, d, f, cfg=None, device=None, dtype=torch.float32, std=0.02):
        super().__init__()
        self.cfg = cfg or MLPConfig()
        self.w1 = torch.nn.Parameter(torch.randn(2 * f, d, device=device, dtype=dtype) * std)
        self.w2 = torch.nn.Parameter(torch.randn(d, f, device=device, dtype=dtype) * std)

    def forward(self, x):
        return FP8MLPFunction.apply(x, self.w1, self.w2, self.cfg)
