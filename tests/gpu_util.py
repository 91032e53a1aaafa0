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


# |x| at or above which round-to-nearest-even to fp32 gives an infinity
FP32_OVERFLOW = 2.0 ** 128 - 2.0 ** 103
# half the fp32 spacing below 2^-126 (the smallest subnormal is 2^-149)
HALF_SUBNORMAL = 2.0 ** -150


def check_gemm(got, ref, bound, what, rel=1e-5, extra=0.0):
    """The products' tolerance, elementwise, against the oracle's fp64 result
    ref and bound = 2^-(ba+bb) * sum |a||b|:
      * where ref is NaN (a NaN code among the output's terms, inf * 0,
        inf - inf) the output must be NaN; where ref is +-inf, that infinity;
      * otherwise |got - ref| <= rel * bound + 2^-150: the second term is half
        the fp32 spacing below 2^-126, what the output's own rounding can cost
        where the exact result lies in fp32's subnormal range or below;
      * an infinity of ref's sign is also accepted where |ref| + rel * bound
        reaches fp32's overflow threshold (results beyond fp32's range).
    extra (scalar or elementwise) widens the finite bar by further rounding
    the operation is allowed, e.g. the fp32 addition of an accumulating
    product.  Returns the worst err / bound over the finite, in-range
    outputs, beyond HALF_SUBNORMAL + extra."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    nan_ref, inf_ref = np.isnan(ref), np.isinf(ref)
    fin = ~(nan_ref | inf_ref)
    reffin = np.where(fin, ref, 0.0)
    bndfin = np.where(fin, bound, 0.0)
    extra = np.where(fin, np.asarray(extra, dtype=np.float64), 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.abs(got - reffin)
        ok_fin = fin & (err <= rel * bndfin + HALF_SUBNORMAL + extra)
        overflow = fin & np.isinf(got) & (np.sign(got) == np.sign(reffin)) & \
            (np.abs(reffin) + rel * bndfin >= FP32_OVERFLOW)
        ok = np.where(nan_ref, np.isnan(got),
                      np.where(inf_ref, got == ref, ok_fin | overflow))
        inrange = fin & np.isfinite(got)
        excess = np.maximum(err - HALF_SUBNORMAL - extra, 0.0)   # beyond the output's own rounding
        ratio = np.where(inrange & (bndfin > 0), excess / np.where(bndfin > 0, bndfin, 1.0),
                         np.where(inrange & (excess > 0), np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    if not ok.all():
        idx = np.argwhere(~ok)
        i = tuple(idx[0])
        raise AssertionError(f"{what}: {len(idx)} of {ok.size} outside the bound; first at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}; worst err/bound {worst:.3e}")
    return worst
