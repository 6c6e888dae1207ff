"""Shared helpers of the GPU parity tests: device transfer, exact bf16
handling, and oracle evaluation on sampled tokens / experts of a full-size
layer."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O

DEV = torch.device("cuda:0")

# Tolerances (relative Frobenius error).
TOL_BF16 = 1e-2   # bf16 storage, fp32 accumulation (layer outputs and grads)
TOL_F32 = 1e-5    # float32 path, and every float32 gate weight / probability
# A bf16 tensor produced by ONE rounding of an fp32 value that is itself
# accurate to ~1e-6 has per-element relative error <= 2^-9 ~ 1.95e-3, so its
# relative Frobenius error is below that; 2.5e-3 leaves room for the fp32 part.
TOL_ONE_ROUNDING = 2.5e-3
# Router logits: float32 sums of exactly representable products (bf16 x bf16,
# or float32 inputs), so their only error is float32 accumulation rounding
# (~sqrt(#terms) * 2^-24 relative to the partial sums: ~1e-6 at d = 4096).
TOL_LOGITS = 1e-5
# A routing difference counts as a near tie when the picked expert's score is
# within this fraction of the token's largest |score| of the score it replaces.
NEAR_TIE = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    """Host array -> device tensor.  float arrays go to ``dtype`` (float32 or
    bfloat16; values must already be representable), ints stay int32."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype in (torch.int32, torch.int64):
        return t.to(torch.int32).to(DEV).contiguous()
    t = t.to(torch.float32)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV).contiguous()


def host(t):
    """Device tensor -> float64 (floats) or int (ints) NumPy array."""
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    a = t.cpu().numpy()
    return a.astype(np.float64) if a.dtype.kind == "f" else a


def bits(t):
    """Raw 16-bit patterns of a bf16 tensor as int16 NumPy array."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy()


def rel(got, ref):
    return O.rel_fro(got, ref)


# ------------------------------------------------------------------ comparisons
def routing_flips(idx, z, k):
    """Tokens whose selected ids ``idx [T,k]`` differ from the oracle's top-k of
    the float64 scores ``z [T,E]``, and those among them that are NOT near
    ties.  A token is a near tie when its ids are distinct and, for every slot
    j, the score (in ``z``) of its j-th id is within NEAR_TIE * max|z[t]| of
    the j-th largest score: the two selections then differ only by the
    rounding of scores that are equal to that accuracy."""
    oi = O.topk_experts(z, k)
    diff = np.flatnonzero((np.asarray(idx) != oi).any(axis=1))
    bad = []
    for t in diff:
        zt = np.asarray(z[t], np.float64)
        ranked = -np.sort(-zt)[:k]
        eps = NEAR_TIE * np.max(np.abs(zt))
        ids = np.asarray(idx[t])
        if len(set(ids.tolist())) != k or np.any(np.abs(zt[ids] - ranked) > eps):
            bad.append(int(t))
    return diff, bad


def rel_by_expert(dev_t, ref, cols=slice(None)):
    """Relative Frobenius error of a device tensor ``[E, R, C]`` (any float
    dtype) against ``ref`` over columns ``cols``, one expert at a time, so
    that no float64 copy of the whole device tensor is made."""
    num = den = 0.0
    for e in range(ref.shape[0]):
        g = host(dev_t[e])[:, cols]
        r = np.asarray(ref[e], np.float64)[:, cols]
        num += float(np.sum((g - r) ** 2))
        den += float(np.sum(r ** 2))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(np.sqrt(num / den))
