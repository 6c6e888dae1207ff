"""CPU oracle of the sparse mixture-of-experts layer.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  The GPU library never calls it, and the two share
no code: no kernels, headers, tables or helpers.

What it computes: one MoE layer on one device's share of T tokens, forward
and backward, written out as the plain definition in float64 NumPy.  No
blocking, fusion or reordering beyond what the definition states; a library
matmul or sort serves as a single step where one is used.

Sources, cited by page title and section:

* [Brief]   llm-wiki paper brief of arXiv 2604.00785, "在 Aurora 超级计算机上
  实现大规模 MoE 语言模型的可扩展预训练" (Scalable pretraining of large MoE
  language models on the Aurora supercomputer).
* [Summary] shd-paper.top summary "Scalable Pretraining of Large Mixture of
  Experts Language Models on Aurora Super Computer".

The pages name the steps of the expert computation -- expert selection in the
forward pass [Summary, Method details / technical framework]; GPU kernels for
token counting and index generation, and a grouped GEMM that merges all
experts' matrix products [Brief, Core method]; optimised matmul and
activation implementations [Summary, Method details / key design]; a forward
plus backward pass as the unit that is sped up [Brief, Key results] -- but
define none of them formally.  Readings taken where they are silent:

R1  Gate: softmax over all E experts of the (optionally biased) router
    logits; the k experts with the largest logits are selected; their softmax
    probabilities are the combine weights, not renormalised unless
    ``renorm`` is set.
R2  Selection is made on the logits themselves, in the logits' own precision
    (softmax is monotone, so the set equals the top-k of the probabilities).
R3  Slot j of a token holds its j-th largest logit; equal logits go to the
    lower expert index.
R4  Inside an expert's group, slots keep their flat token-major order
    s = t*k + j (a stable sort of the flat expert ids).
R5  Dropless: no capacity limit; every one of the T*k slots is computed.
R6  No biases in the router or the expert FFNs.  An optional per-expert logit
    bias is a fixed input: it shifts selection and probabilities and receives
    no gradient.
R7  Expert FFN = SwiGLU: H = Xp @ W1[e] with W1[e] of shape [d, 2F]; columns
    [0, F) are the gate G, [F, 2F) the up projection U;
    A = silu(G) * U with silu(z) = z * sigmoid(z); Yp = A @ W2[e], W2[e] of
    shape [F, d].
R8  Combine: y[t] = sum_j w[t, j] * Yp[dest[t*k + j]].
R9  A forced assignment (forced uniform routing, [Brief, Limitations]) replaces
    the selected ids; its weights are the softmax probabilities of the forced
    experts, in the forced order.
R10 Backward of L = <y, dy>: the closed forms of each step (chain rule),
    computed without intermediate rounding.

Every function here is pinned by the CPU tests against brute force,
library routines on special cases, closed forms, invariants, or central
finite differences of the forward pass.
"""
from __future__ import annotations

import contextlib

import numpy as np

F64 = np.float64
# Working precision of every step: float64, the precision the oracle is
# pinned and compared in.  ``precision`` switches it (float32 for the CPU
# throughput baseline) without changing any definition.
FT = np.float64


@contextlib.contextmanager
def precision(dtype):
    """Evaluate the oracle's steps in ``dtype`` (e.g. ``np.float32``) inside
    the block.  Only the dtype of the arrays changes; the definitions, the
    order of the steps and the library routines are the same.  Not
    thread-safe (module state)."""
    global FT
    old = FT
    FT = np.dtype(dtype).type
    try:
        yield
    finally:
        FT = old


# --------------------------------------------------------------------------
# Forward: routing  [Summary, Method details / technical framework]
# --------------------------------------------------------------------------
def router_logits(x, wr):
    """Router logits ``L[t, e] = sum_i x[t, i] * wr[i, e]`` in float64."""
    return np.asarray(x, FT) @ np.asarray(wr, FT)


def biased_logits(logits, bias):
    """Selection scores ``z = L + bias`` (R6), computed in the logits' dtype.

    The addition is done in the precision of ``logits`` (float32 logits give a
    float32 sum) so that the selection decision of R2 is taken in the same
    precision as the logits it is given.
    """
    logits = np.asarray(logits)
    if bias is None:
        return logits
    return logits + np.asarray(bias).astype(logits.dtype)


def softmax(z):
    """Row softmax ``p[t, e] = exp(z[t, e]) / sum_e' exp(z[t, e'])`` (R1).

    The row maximum is subtracted first; this leaves the value unchanged.
    """
    z = np.asarray(z, FT)
    m = z.max(axis=-1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=-1, keepdims=True)


def topk_experts(z, k):
    """The k largest entries of each row of ``z`` (R2, R3).

    Returns int32 ``[T, k]``: column j is the expert with the j-th largest
    score; equal scores are ordered by increasing expert index (a stable sort
    of ``-z``).
    """
    z = np.asarray(z)
    order = np.argsort(-z, axis=-1, kind="stable")
    return np.ascontiguousarray(order[:, :k]).astype(np.int32)


def gate_weights(p, idx, renorm=False):
    """Combine weights ``w[t, j] = p[t, idx[t, j]]`` (R1), optionally divided
    by their sum over j."""
    w = np.take_along_axis(np.asarray(p, FT), np.asarray(idx, np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def route(logits, k, bias=None, forced_idx=None, renorm=False):
    """Expert selection: ``(idx int32[T,k], w f64[T,k], p f64[T,E])``.

    R1-R3, R6, R9.  ``logits`` may be float32 (as produced by a device) or
    float64; the selection is taken on ``logits + bias`` in that precision.
    """
    z = biased_logits(logits, bias)
    p = softmax(z)
    if forced_idx is not None:
        idx = np.ascontiguousarray(forced_idx, dtype=np.int32)
    else:
        idx = topk_experts(z, k)
    return idx, gate_weights(p, idx, renorm), p


# --------------------------------------------------------------------------
# Forward: token counting and index generation  [Brief, Core method]
# --------------------------------------------------------------------------
def count_tokens(idx, E):
    """``counts[e]`` = number of slots (t, j) whose expert is e."""
    flat = np.asarray(idx).reshape(-1)
    return np.array([np.count_nonzero(flat == e) for e in range(E)],
                    dtype=np.int32)


def build_index(idx, E):
    """Per-expert offsets and the slot <-> row maps of the expert-sorted order.

    Returns ``(counts, offsets, dest, src)``:

    * ``offsets[E+1]``: exclusive prefix sum of ``counts``; expert e owns rows
      ``[offsets[e], offsets[e+1])`` of the permuted buffers.
    * ``src[p]``: the flat slot ``s = t*k + j`` that row p holds; inside an
      expert's rows, slots appear in increasing s (R4).
    * ``dest[s]``: the row of slot s, i.e. the inverse of ``src``.
    """
    flat = np.asarray(idx).reshape(-1)
    Tk = flat.size
    counts = count_tokens(idx, E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    src = np.empty(Tk, dtype=np.int32)
    for e in range(E):
        src[offsets[e]:offsets[e + 1]] = np.flatnonzero(flat == e)
    dest = np.empty(Tk, dtype=np.int32)
    dest[src] = np.arange(Tk, dtype=np.int32)
    return counts, offsets, dest, src


def permute(x, src, k):
    """Expert-sorted copy of the token rows: ``xp[p] = x[src[p] // k]``."""
    return np.asarray(x)[np.asarray(src) // k]


# --------------------------------------------------------------------------
# Forward: grouped GEMM and activation  [Brief, Core method]; [Summary,
# Method details / key design]
# --------------------------------------------------------------------------
def grouped_matmul(a, w, offsets):
    """One matrix product per expert: rows of e times ``w[e]``.

    ``a[M, K]`` expert-sorted rows, ``w[E, K, N]``; returns ``c[M, N]`` with
    ``c[offsets[e]:offsets[e+1]] = a[offsets[e]:offsets[e+1]] @ w[e]``.
    """
    a = np.asarray(a, FT)
    E, K, N = w.shape
    c = np.zeros((a.shape[0], N), dtype=FT)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            c[r0:r1] = a[r0:r1] @ np.asarray(w[e], FT)
    return c


def sigmoid(z):
    """Logistic function 1 / (1 + exp(-z)), overflow-free form."""
    z = np.asarray(z, FT)
    return np.exp(-np.logaddexp(0.0, -z))


def silu(z):
    """SiLU (swish) ``z * sigmoid(z)``."""
    z = np.asarray(z, FT)
    return z * sigmoid(z)


def swiglu(h):
    """Gated activation of R7: ``A = silu(G) * U`` with ``G, U = h[:, :F],
    h[:, F:]``."""
    h = np.asarray(h, FT)
    F = h.shape[1] // 2
    return silu(h[:, :F]) * h[:, F:]


def combine(yp, dest, w, k):
    """Weighted un-permute (R8): ``y[t] = sum_j w[t, j] * yp[dest[t*k + j]]``."""
    yp = np.asarray(yp, FT)
    w = np.asarray(w, FT)
    T = w.shape[0]
    d2 = np.asarray(dest).reshape(T, k)
    y = np.zeros((T, yp.shape[1]), dtype=FT)
    for j in range(k):
        y += w[:, j:j + 1] * yp[d2[:, j]]
    return y


def layer_forward(x, wr, w1, w2, k, bias=None, forced_idx=None, renorm=False,
                  logits=None):
    """Whole forward pass; returns every intermediate in a dict.

    ``logits`` may be supplied (e.g. a device's float32 router output) to take
    the routing decision on exactly those values; otherwise they are
    ``x @ wr`` in float64.
    """
    x = np.asarray(x, FT)
    T = x.shape[0]
    E = w1.shape[0]
    if logits is None:
        logits = router_logits(x, wr)
    idx, w, p = route(logits, k, bias, forced_idx, renorm)
    counts, offsets, dest, src = build_index(idx, E)
    xp = permute(x, src, k)
    h = grouped_matmul(xp, w1, offsets)
    a = swiglu(h)
    yp = grouped_matmul(a, w2, offsets)
    y = combine(yp, dest, w, k)
    assert y.shape == (T, x.shape[1])
    return dict(logits=logits, idx=idx, w=w, p=p, counts=counts,
                offsets=offsets, dest=dest, src=src, xp=xp, h=h, a=a, yp=yp,
                y=y)


# --------------------------------------------------------------------------
# Backward of L = <y, dy>  (R10)  [Brief, Key results: forward plus backward]
# --------------------------------------------------------------------------
def combine_backward(dy, yp, dest, w, k):
    """Gradients of R8: ``dyp[dest[t*k+j]] = w[t, j] * dy[t]`` and
    ``dw[t, j] = <dy[t], yp[dest[t*k+j]]>``."""
    dy = np.asarray(dy, FT)
    yp = np.asarray(yp, FT)
    w = np.asarray(w, FT)
    T = dy.shape[0]
    d2 = np.asarray(dest).reshape(T, k)
    dyp = np.zeros_like(yp)
    dw = np.zeros((T, k), dtype=FT)
    for j in range(k):
        dyp[d2[:, j]] = w[:, j:j + 1] * dy
        dw[:, j] = np.sum(dy * yp[d2[:, j]], axis=1)
    return dyp, dw


def grouped_matmul_backward(a, w, dc, offsets):
    """Gradients of ``grouped_matmul``: per expert e,
    ``da_e = dc_e @ w[e]^T`` and ``dw[e] = a_e^T @ dc_e`` (zero for an expert
    with no rows)."""
    a = np.asarray(a, FT)
    dc = np.asarray(dc, FT)
    E, K, N = w.shape
    da = np.zeros((a.shape[0], K), dtype=FT)
    dw = np.zeros((E, K, N), dtype=FT)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            we = np.asarray(w[e], FT)
            da[r0:r1] = dc[r0:r1] @ we.T
            dw[e] = a[r0:r1].T @ dc[r0:r1]
    return da, dw


def swiglu_backward(h, da):
    """Gradient of ``swiglu``: with s = sigmoid(G),
    ``dG = da * U * s * (1 + G * (1 - s))`` and ``dU = da * G * s``."""
    h = np.asarray(h, FT)
    da = np.asarray(da, FT)
    F = h.shape[1] // 2
    g, u = h[:, :F], h[:, F:]
    s = sigmoid(g)
    dg = da * u * s * (1.0 + g * (1.0 - s))
    du = da * g * s
    return np.concatenate([dg, du], axis=1)


def permute_backward(dxp, dest, k, T):
    """Gradient of ``permute``: ``dx[t] = sum_j dxp[dest[t*k + j]]``."""
    dxp = np.asarray(dxp, FT)
    d2 = np.asarray(dest).reshape(T, k)
    dx = np.zeros((T, dxp.shape[1]), dtype=FT)
    for j in range(k):
        dx += dxp[d2[:, j]]
    return dx


def gate_backward(p, idx, dw, renorm=False):
    """Gradient of the router logits from the combine-weight gradient.

    First the gradient of the selected probabilities (with ``renorm``,
    ``w_j = p_j / S``, ``S = sum_j p_j`` gives
    ``dp_j = (dw_j - sum_l dw_l w_l) / S``), scattered into ``dp[T, E]``;
    then the softmax Jacobian: ``dz = p * (dp - <p, dp>)``.
    """
    p = np.asarray(p, FT)
    dw = np.asarray(dw, FT)
    idx = np.asarray(idx, np.int64)
    T, E = p.shape
    if renorm:
        pk = np.take_along_axis(p, idx, axis=1)
        S = pk.sum(axis=1, keepdims=True)
        wn = pk / S
        dpk = (dw - np.sum(dw * wn, axis=1, keepdims=True)) / S
    else:
        dpk = dw
    dp = np.zeros((T, E), dtype=FT)
    rows = np.repeat(np.arange(T), idx.shape[1])
    np.add.at(dp, (rows, idx.reshape(-1)), dpk.reshape(-1))
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def router_backward(x, wr, dz):
    """Gradients of ``router_logits``: ``dx = dz @ wr^T``, ``dwr = x^T @ dz``."""
    x = np.asarray(x, FT)
    wr = np.asarray(wr, FT)
    dz = np.asarray(dz, FT)
    return dz @ wr.T, x.T @ dz


def layer_backward(fwd, dy, x, wr, w1, w2, k, renorm=False):
    """Whole backward pass from the dict of ``layer_forward``.

    Returns a dict with ``dx``, ``dwr``, ``dw1``, ``dw2`` and the
    intermediates ``dyp, dw, da, dh, dxp, dz``.
    """
    dy = np.asarray(dy, FT)
    T = dy.shape[0]
    dyp, dw = combine_backward(dy, fwd["yp"], fwd["dest"], fwd["w"], k)
    da, dw2 = grouped_matmul_backward(fwd["a"], w2, dyp, fwd["offsets"])
    dh = swiglu_backward(fwd["h"], da)
    dxp, dw1 = grouped_matmul_backward(fwd["xp"], w1, dh, fwd["offsets"])
    dx_experts = permute_backward(dxp, fwd["dest"], k, T)
    dz = gate_backward(fwd["p"], fwd["idx"], dw, renorm)
    dx_router, dwr = router_backward(x, wr, dz)
    return dict(dx=dx_experts + dx_router, dwr=dwr, dw1=dw1, dw2=dw2,
                dyp=dyp, dw=dw, da=da, dh=dh, dxp=dxp, dz=dz,
                dx_experts=dx_experts)


def rel_fro(got, ref):
    """Relative Frobenius error ``||got - ref||_F / ||ref||_F`` (0 if both are
    zero)."""
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    num = np.linalg.norm((got - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
