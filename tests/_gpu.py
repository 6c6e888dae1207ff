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


# ------------------------------------------------------------------ sampling
def sample_tokens(inp, gpu_logits, k, tokens, renorm=False):
    """Oracle forward+backward of the given tokens only (tokens are
    independent in the forward pass and in dx), routed on the device's fp32
    logits of those tokens.  Returns (fwd, bwd) dicts of the sub-problem:
    y, dx, dz (= dlogits), w, idx are exact for these tokens."""
    t = np.asarray(tokens)
    forced = None if inp.forced_idx is None else inp.forced_idx[t]
    fwd = O.layer_forward(inp.x[t], inp.wr, inp.w1, inp.w2, k, bias=inp.bias, forced_idx=forced,
                          renorm=renorm, logits=gpu_logits[t])
    bwd = O.layer_backward(fwd, inp.dy[t], inp.x[t], inp.wr, inp.w1, inp.w2, k, renorm=renorm)
    return fwd, bwd


def expert_weight_grads(inp, k, idx, w, e):
    """Oracle dW1[e], dW2[e] from every slot routed to expert e (routing
    idx/w given), composed from the oracle's per-step functions on the
    one-expert sub-problem."""
    flat = idx.reshape(-1)
    slots = np.flatnonzero(flat == e)
    tok = slots // k
    n = len(slots)
    off = np.array([0, n])
    w1 = inp.w1[e:e + 1]
    w2 = inp.w2[e:e + 1]
    xp = inp.x[tok].astype(np.float64)
    wt = w.reshape(-1)[slots][:, None]
    h = O.grouped_matmul(xp, w1, off)
    a = O.swiglu(h)
    dyp = wt * inp.dy[tok].astype(np.float64)
    da, dw2 = O.grouped_matmul_backward(a, w2, dyp, off)
    dh = O.swiglu_backward(h, da)
    _, dw1 = O.grouped_matmul_backward(xp, w1, dh, off)
    return dw1[0], dw2[0], n
