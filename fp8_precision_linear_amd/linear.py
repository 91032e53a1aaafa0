"""The FP8-AMAX linear layer as a PyTorch autograd Function and module.

"Training and inference of large language models using 8-bit floating point",
review page, "Proposed method": the input, the weight and the output gradient
each get a per-tensor power-of-two scale from their amax (bullets 1-2), are
cast to E4M3 (input, weight) or E5M2 (gradient) (bullet 4), and the three
products run in FP8 and are unscaled afterwards (bullet 3), in training
(bullet 5):
    forward   y  = x8 . w8^T            (fp8_scaled_gemm_fwd)
    backward  dx = dy8 . w8             (fp8_scaled_gemm_dgrad)
              dw = dy8^T . x8           (fp8_scaled_gemm_wgrad)
x may have any leading dimensions ([..., K]); w is [N, K].  Outputs and
gradients are fp32 (autograd converts dx to x's dtype).

Products whose outputs have too few tiles to fill the GPU (a small batch of
tokens) run split along the contraction (fp8_scaled_gemm_ws).

Scaling modes (ScalingState):
  * "current": every quantisation is amax -> compute_bias -> cast on the
    tensor itself, as the method states (one fp8_quantize call, which makes
    them in one launch for small tensors and three for large ones);
  * "delayed": the bias of a tensor comes from the amax its previous step's
    quantisation returned, and the cast returns this step's amax in the same
    pass (one fp8_quantize_delayed call, which overwrites the previous amax
    with the new one), so each quantisation reads its input once; the first
    step of each tensor uses "current".  Values beyond the previous
    step's scale saturate: the pages' delayed / infrequent bias update trades
    that for the skipped amax pass.
Every bias is logged per tensor (BiasLog), without a host synchronisation.
For post-training-quantised inference (bullet 5) FP8Linear.freeze_weight()
quantises the weight once; later calls reuse its codes and bias.

With FP8Linear(..., fuse_wgrad_accumulation=True) the weight gradient of a
backward pass is added straight into weight.grad by
fp8_scaled_gemm_accumulate (one fp32 addition per element), so micro-batches
accumulate without a separate fp32 gradient per pass; the first pass after
weight.grad was cleared (None) writes it.  The weight must be an fp32 master.
"""
import torch

from . import (E4M3, E5M2, MATH_EXACT, OP_DGRAD, OP_FWD, OP_WGRAD, quantize, quantize_delayed,
               scaled_gemm_accumulate, scaled_gemm_auto)

ROLES = ("x", "w", "dy")
FORMATS = {"x": E4M3, "w": E4M3, "dy": E5M2}


class ScalingState:
    """Per-tensor scaling of one linear layer: margins, the mode ("current" or
    "delayed"), each role's amax from its last quantisation (device
    float32[1]), and an optional bias log (mlp.BiasLog)."""

    def __init__(self, mode="current", margins=None, math=MATH_EXACT, log=None):
        if mode not in ("current", "delayed"):
            raise ValueError(f"mode is 'current' or 'delayed', got {mode!r}")
        self.mode = mode
        self.fuse_wgrad_accumulation = False
        self.margins = {r: 0 for r in ROLES}
        self.margins.update(margins or {})
        self.math = math
        self.log = log
        self.amax = {}
        self.frozen = {}   # role -> (codes, bias) reused instead of quantising

    def freeze(self, role, t):
        """Quantise t for `role` once (current scaling); later quantise()
        calls for that role return these codes and bias."""
        self.frozen.pop(role, None)
        self.frozen[role] = self.quantise(role, t)

    def unfreeze(self, role):
        self.frozen.pop(role, None)

    def quantise(self, role, t):
        """(codes, bias) of tensor t for `role`."""
        if role in self.frozen:
            return self.frozen[role]
        fmt, margin = FORMATS[role], self.margins[role]
        prev = self.amax.get(role)
        if self.mode == "delayed" and prev is not None:
            codes, bias = quantize_delayed(t, fmt, prev, margin)  # prev now holds this step's amax
            amax = prev
        else:
            codes, bias, amax = quantize(t, fmt, margin)
        self.amax[role] = amax
        if self.log is not None:
            self.log.record(role, bias)
        return codes, bias


def _flat(t):
    return t.contiguous().reshape(-1, t.shape[-1])



class FP8LinearFunction(torch.autograd.Function):
    """y = x . w^T with FP8-AMAX products; gradients for x and w."""

    @staticmethod
    def forward(ctx, x, w, state):
        if w.dim() != 2 or x.shape[-1] != w.shape[1]:
            raise ValueError(f"x [..., K] and w [N, K] do not match: {tuple(x.shape)}, {tuple(w.shape)}")
        x2 = _flat(x)
        x8, bx = state.quantise("x", x2)
        w8, bw = state.quantise("w", w.contiguous())
        y = scaled_gemm_auto(OP_FWD, x8, E4M3, bx, w8, E4M3, bw, math=state.math)
        ctx.saved = (x8, bx, w8, bw)
        ctx.state = state
        ctx.weight = w
        ctx.x_shape = x.shape
        return y.reshape(*x.shape[:-1], w.shape[0])

    @staticmethod
    def backward(ctx, dy):
        x8, bx, w8, bw = ctx.saved
        state = ctx.state
        dy8, bdy = state.quantise("dy", _flat(dy))
        dx = scaled_gemm_auto(OP_DGRAD, dy8, E5M2, bdy, w8, E4M3, bw, math=state.math)
        w = ctx.weight
        if state.fuse_wgrad_accumulation and w.grad is not None:
            # weight.grad += dW in the product's epilogue; autograd gets no
            # weight gradient to add
            scaled_gemm_accumulate(OP_WGRAD, dy8, E5M2, bdy, x8, E4M3, bx, w.grad, math=state.math)
            dw = None
        else:
            dw = scaled_gemm_auto(OP_WGRAD, dy8, E5M2, bdy, x8, E4M3, bx, math=state.math)
        ctx.saved = None
        ctx.weight = None
        return dx.reshape(ctx.x_shape), dw, None


class FP8Linear(torch.nn.Module):
    """Linear layer without bias whose three products are FP8-AMAX scaled
    GEMMs; the weight (out_features x in_features) is an fp32 master by
    default."""

    def __init__(self, in_features, out_features, mode="current", margins=None, math=MATH_EXACT,
                 log=None, device=None, dtype=torch.float32, std=0.02, fuse_wgrad_accumulation=False):
        super().__init__()
        if fuse_wgrad_accumulation and dtype != torch.float32:
            raise ValueError("fused weight-gradient accumulation needs an fp32 weight")
        self.state = ScalingState(mode, margins, math, log)
        self.state.fuse_wgrad_accumulation = fuse_wgrad_accumulation
        self.weight = torch.nn.Parameter(torch.randn(out_features, in_features, device=device,
                                                     dtype=dtype) * std)

    def forward(self, x):
        return FP8LinearFunction.apply(x, self.weight, self.state)

    @torch.no_grad()
    def freeze_weight(self):
        """Post-training quantisation: the weight's codes and bias are made
        now, from its current values, and reused by every later call until
        unfreeze_weight() (the weight gradient is still computed)."""
        mode, self.state.mode = self.state.mode, "current"
        try:
            self.state.freeze("w", self.weight.detach().contiguous())
        finally:
            self.state.mode = mode

    def unfreeze_weight(self):
        self.state.unfreeze("w")
