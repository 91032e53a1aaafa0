"""Helpers shared by the GPU parity tests (device tensors <-> numpy words)."""
import sys

import numpy as np
import torch


def say(*a):
    """Name the case before a GPU step, flushed, so a lost run still shows it."""
    print("[case]", *a, file=sys.stderr, flush=True)


def need_gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a HIP device"
    import fp8_precision_linear_amd as fl
    return fl


def bf16_dev(words):
    return torch.from_numpy(np.ascontiguousarray(words).astype(np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def f32_dev(words):
    return torch.from_numpy(np.ascontiguousarray(words).astype(np.uint32).view(np.float32)).cuda()


def words_of(t):
    """numpy words of a CPU or device tensor (uint16 for bf16, uint32 for fp32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    raise TypeError(t.dtype)


def i32_dev(v):
    return torch.tensor([int(v)], dtype=torch.int32, device="cuda")


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def check_gemm(got, ref, bound, what, rel=1e-5):
    """|got - ref| <= rel * bound elementwise (bound = sum |a||b| * 2^-(ba+bb));
    reports the worst element and the worst err/bound ratio."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    ok = err <= rel * bound
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    if not ok.all():
        idx = np.argwhere(~ok)
        i = tuple(idx[0])
        raise AssertionError(f"{what}: {len(idx)} of {ok.size} outside the bound; first at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}; worst err/bound {worst:.3e}")
    return worst
