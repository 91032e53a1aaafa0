"""Seeded synthetic inputs and the workload table for the FP8-AMAX linear layer.

This module holds no step of the method (no amax, bias, cast or matmul): it
only draws the bf16 tensors that the HIP library and the CPU oracle are both
fed, and lists which products each workload runs.  The tests, the smoke check
and the benchmark use it; it imports neither the oracle nor the HIP binding.

The workloads stand in for the pages' fine-tuning and inference runs of GPT and
Llama 2 models from 111M to 70B parameters ("Training and inference of large
language models using 8-bit floating point", review page, one-sentence summary
and "Main findings"): the datasets and trained weights are not used, only each
model family's linear-layer shapes with seeded random values.

Recipe: numpy PCG64, ``np.random.default_rng(1000 * workload + t)`` where t is
the tensor's position in the workload's tensor list; normals are
``standard_normal(dtype=float32) * sigma``; Student-t(3) values are drawn in
float64 and narrowed to float32, then 0.1% of positions (drawn without
replacement) are multiplied by 100; float32 is rounded to bf16 (nearest-even)
by torch.
"""
from dataclasses import dataclass, field
import hashlib

import numpy as np
import torch

E4M3, E5M2 = 0, 1


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: tuple
    dist: str          # "normal" or "t3_outliers"
    sigma: float
    fmt: int           # E4M3 or E5M2
    margin: int
    timed: bool        # quantised inside the timed step (dynamic) or beforehand (static)


@dataclass(frozen=True)
class LinearSpec:
    name: str
    x: str             # input activation, [M x K]
    w: str             # weight, [N x K]
    dy: str            # output gradient, [M x N], or "" for forward-only
    M: int
    N: int
    K: int
    passes: tuple      # subset of ("fwd", "dgrad", "wgrad")


@dataclass(frozen=True)
class Workload:
    index: int         # 1-based workload number, also the seed base
    name: str
    tensors: tuple     # TensorSpec, in seed order
    linears: tuple     # LinearSpec, in the step's launch order
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def tensor(self, name):
        for t in self.tensors:
            if t.name == name:
                return t
        raise KeyError(name)

    def seed(self, name):
        for i, t in enumerate(self.tensors):
            if t.name == name:
                return 1000 * self.index + i
        raise KeyError(name)

    def flops(self):
        return sum(2 * l.M * l.N * l.K * len(l.passes) for l in self.linears)


def _single_linear():
    t = (TensorSpec("X", (128, 256), "normal", 1.0, E4M3, 0, True),
         TensorSpec("W", (256, 256), "normal", 0.02, E4M3, 0, True))
    l = (LinearSpec("linear", "X", "W", "", 128, 256, 256, ("fwd",)),)
    return Workload(1, "single-linear-fwd-128x256x256", t, l)


def _gpt111m():
    M = 2048
    shapes = (("qkv", 768, 2304), ("up", 768, 3072), ("down", 3072, 768))
    ts, ls = [], []
    for name, K, N in shapes:
        ts += [TensorSpec(f"X_{name}", (M, K), "normal", 1.0, E4M3, 0, True),
               TensorSpec(f"W_{name}", (N, K), "normal", 0.02, E4M3, 0, True),
               TensorSpec(f"dY_{name}", (M, N), "normal", 1e-3, E5M2, 0, True)]
        ls.append(LinearSpec(name, f"X_{name}", f"W_{name}", f"dY_{name}", M, N, K,
                             ("fwd", "dgrad", "wgrad")))
    return Workload(2, "gpt-111m-layer-fwd-bwd-tokens2048-hidden768", tuple(ts), tuple(ls))


def _llama7b_mlp():
    M, H, F = 4096, 4096, 11008
    ts = (TensorSpec("X", (M, H), "t3_outliers", 1.0, E4M3, 1, True),
          TensorSpec("H", (M, F), "t3_outliers", 1.0, E4M3, 1, True),
          TensorSpec("W_gate", (F, H), "normal", 0.02, E4M3, 1, True),
          TensorSpec("W_up", (F, H), "normal", 0.02, E4M3, 1, True),
          TensorSpec("W_down", (H, F), "normal", 0.02, E4M3, 1, True))
    ls = (LinearSpec("gate", "X", "W_gate", "", M, F, H, ("fwd",)),
          LinearSpec("up", "X", "W_up", "", M, F, H, ("fwd",)),
          LinearSpec("down", "H", "W_down", "", M, H, F, ("fwd",)))
    return Workload(3, "llama2-7b-mlp-fwd-tokens4096", ts, ls)


def _llama13b_bwd():
    M, H, F = 4096, 5120, 13824
    shapes = (("gate", H, F), ("up", H, F), ("down", F, H))
    ts, ls = [], []
    for name, K, N in shapes:
        ts += [TensorSpec(f"dY_{name}", (M, N), "normal", 1e-6, E5M2, 0, True),
               TensorSpec(f"X_{name}", (M, K), "normal", 1.0, E4M3, 0, False),
               TensorSpec(f"W_{name}", (N, K), "normal", 0.02, E4M3, 0, False)]
        ls.append(LinearSpec(name, f"X_{name}", f"W_{name}", f"dY_{name}", M, N, K,
                             ("dgrad", "wgrad")))
    return Workload(4, "llama2-13b-mlp-bwd-tokens4096", tuple(ts), tuple(ls))


def _llama70b_infer():
    M, H, Q, F = 8192, 8192, 10240, 28672
    ts = (TensorSpec("X_qkv", (M, H), "normal", 1.0, E4M3, 0, True),
          TensorSpec("X_o", (M, H), "normal", 1.0, E4M3, 0, True),
          TensorSpec("X_mlp", (M, H), "normal", 1.0, E4M3, 0, True),
          TensorSpec("H", (M, F), "normal", 1.0, E4M3, 0, True),
          TensorSpec("W_qkv", (Q, H), "normal", 0.02, E4M3, 0, False),
          TensorSpec("W_o", (H, H), "normal", 0.02, E4M3, 0, False),
          TensorSpec("W_gate", (F, H), "normal", 0.02, E4M3, 0, False),
          TensorSpec("W_up", (F, H), "normal", 0.02, E4M3, 0, False),
          TensorSpec("W_down", (H, F), "normal", 0.02, E4M3, 0, False))
    ls = (LinearSpec("qkv", "X_qkv", "W_qkv", "", M, Q, H, ("fwd",)),
          LinearSpec("o", "X_o", "W_o", "", M, H, H, ("fwd",)),
          LinearSpec("gate", "X_mlp", "W_gate", "", M, F, H, ("fwd",)),
          LinearSpec("up", "X_mlp", "W_up", "", M, F, H, ("fwd",)),
          LinearSpec("down", "H", "W_down", "", M, H, F, ("fwd",)))
    return Workload(5, "llama2-70b-layer-inference-tokens8192", ts, ls)


WORKLOADS = {w.index: w for w in (_single_linear(), _gpt111m(), _llama7b_mlp(),
                                  _llama13b_bwd(), _llama70b_infer())}


@dataclass(frozen=True)
class ChainedMLP:
    """A gated MLP trained with FP8 products end to end (forward and backward
    through the SwiGLU between them): x [tokens, d] bf16, w1 = [W_gate; W_up]
    [2f, d] and w2 = W_down [d, f] as float32 master weights, and g = dL/dy
    [tokens, d] float32, the upstream gradient of the synthetic loss
    L = sum(y * g)."""
    index: int
    name: str
    tokens: int
    d: int
    f: int
    x_dist: str = "t3_outliers"
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    g_sigma: float = 1e-6

    ORDER = ("X", "W1", "W2", "G")

    def seed(self, name):
        return 1000 * self.index + self.ORDER.index(name)

    def shape(self, name):
        return {"X": (self.tokens, self.d), "W1": (2 * self.f, self.d), "W2": (self.d, self.f),
                "G": (self.tokens, self.d)}[name]

    def flops(self):
        """Six products per step (three forward-shaped, each with a data and a
        weight gradient): 18 * tokens * f * d."""
        return 18 * self.tokens * self.f * self.d


def chained_mlp_tensor(m, name):
    """CPU tensor `name` of chained MLP `m`: X bf16, the rest float32."""
    if name == "X":
        return draw_bf16(m.seed(name), m.shape(name), m.x_dist, m.x_sigma)
    sigma = m.w_sigma if name in ("W1", "W2") else m.g_sigma
    return torch.from_numpy(draw_f32(m.seed(name), m.shape(name), "normal", sigma))


# Llama-2-7B's MLP (hidden 4096, intermediate 11008) over 4096 tokens.
CHAINED_MLPS = {6: ChainedMLP(6, "llama2-7b-mlp-chained-fwd-bwd-tokens4096", 4096, 4096, 11008)}


def draw_f32(seed, shape, dist, sigma):
    """float32 numpy array of the given distribution (see module docstring)."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    if dist == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
    elif dist == "t3_outliers":
        x = rng.standard_t(3, n).astype(np.float32)
        idx = rng.choice(n, n // 1000, replace=False)
        x[idx] *= np.float32(100.0)
    else:
        raise ValueError(dist)
    return x.reshape(shape)


def to_bf16(x_f32):
    """Round a float32 numpy array to a bf16 torch CPU tensor (nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(x_f32)).to(torch.bfloat16)


def draw_bf16(seed, shape, dist="normal", sigma=1.0):
    return to_bf16(draw_f32(seed, shape, dist, sigma))


def workload_tensor(w, name):
    """The bf16 CPU tensor `name` of workload `w`."""
    t = w.tensor(name)
    return draw_bf16(w.seed(name), t.shape, t.dist, t.sigma)


def bf16_words(t):
    """numpy uint16 view of a bf16 CPU tensor's bits."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def sha256(t):
    """SHA-256 of a CPU tensor's bytes."""
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


def special_bf16_words():
    """Every bf16 bit pattern, 0x0000 .. 0xFFFF."""
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)
