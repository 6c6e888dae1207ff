"""Seeded synthetic inputs for the sparse mixture-of-experts layer.

Shared by the tests, the benchmark and the CPU oracle checks.  This module
holds none of the layer's arithmetic: only workload shapes, seeded normal
draws, the rounding of drawn values to the workload's storage type, and the
two routing-regime inputs (a per-expert logit bias and a forced expert
assignment).  Everything it returns is plain NumPy data on the host.

Draws are made in float32, in fixed 4 Mi-element chunks, each chunk from its
own child of ``numpy.random.SeedSequence(seed)``; the values therefore do not
depend on how many threads fill them.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

_CHUNK = 1 << 22  # elements per independently seeded chunk


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, storage type, value scales and routing regime of one layer call.

    ``T`` tokens of width ``d`` are routed to ``k`` of ``E`` experts; each
    expert is a SwiGLU feed-forward block with inner width ``F``.
    ``regime``: ``"natural"`` (routing follows the router logits),
    ``"skew"`` (a fixed per-expert logit bias, log-Zipf in a seeded expert
    rank) or ``"uniform"`` (a forced assignment that gives every expert exactly
    ``T*k/E`` slots).
    """

    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    dtype: str = "bf16"          # "bf16" or "fp32" storage of x, weights, dy
    w_std: float = 0.02          # std of router and expert weights
    seed: int = 0
    regime: str = "natural"
    zipf_s: float = 1.2          # exponent of the skewed regime's bias

    @property
    def Tk(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 layer: parity at a size the oracle finishes instantly.
    "tiny": Workload("tiny", T=256, d=128, E=8, k=2, F=256, dtype="fp32",
                     w_std=0.02, seed=1000),
    # OLMoE-like layer: 4 sequences of 2048 tokens, 64 experts, top-8.
    "olmoe": Workload("olmoe", T=8192, d=2048, E=64, k=8, F=1024,
                      dtype="bf16", w_std=0.02, seed=1001),
    # Same shapes, skewed routing (hottest expert several times the mean).
    "olmoe_skew": Workload("olmoe_skew", T=8192, d=2048, E=64, k=8, F=1024,
                           dtype="bf16", w_std=0.02, seed=1002,
                           regime="skew"),
    # Same shapes, forced-uniform routing (every expert gets T*k/E slots).
    "olmoe_uniform": Workload("olmoe_uniform", T=8192, d=2048, E=64, k=8,
                              F=1024, dtype="bf16", w_std=0.02, seed=1012,
                              regime="uniform"),
    # Large-expert layer: high FLOP count per call.
    "large": Workload("large", T=16384, d=4096, E=128, k=8, F=1536,
                      dtype="bf16", w_std=0.01, seed=1003),
    # Sparse small groups: 256 experts, ~16 slots each on average.
    "sparse": Workload("sparse", T=512, d=2048, E=256, k=8, F=768,
                       dtype="bf16", w_std=0.02, seed=1004),
}


@dataclasses.dataclass
class Inputs:
    """Host arrays for one layer call.

    Float tensors are float32 arrays whose values are exactly representable in
    the workload's storage type (bf16-rounded for ``dtype == "bf16"``), so the
    GPU path and the oracle consume identical numbers.
    Layouts (row-major): ``x[T,d]``, ``wr[d,E]``, ``w1[E,d,2F]`` (columns
    ``[0,F)`` gate, ``[F,2F)`` up), ``w2[E,F,d]``, ``dy[T,d]``; ``bias[E]``
    float32 or None; ``forced_idx[T,k]`` int32 or None.
    """

    wl: Workload
    x: np.ndarray
    wr: np.ndarray
    w1: np.ndarray
    w2: np.ndarray
    dy: np.ndarray
    bias: Optional[np.ndarray]
    forced_idx: Optional[np.ndarray]


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), in place.

    Returns the same float32 array, now holding bf16-representable values.
    Inputs are finite by construction (normal draws), so NaN handling is not
    needed.
    """
    assert a.dtype == np.float32 and a.flags.c_contiguous
    flat = a.reshape(-1)
    u = flat.view(np.uint32)

    def work(i):
        s = slice(i * _CHUNK, (i + 1) * _CHUNK)
        v = u[s]
        lsb = (v >> np.uint32(16)) & np.uint32(1)
        v += np.uint32(0x7FFF) + lsb
        v &= np.uint32(0xFFFF0000)

    _parallel(work, _nchunks(flat.size))
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-representable float32 values, as uint16."""
    assert a.dtype == np.float32
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _nchunks(n: int) -> int:
    return max(1, (n + _CHUNK - 1) // _CHUNK)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _parallel(fn, n):
    if n == 1:
        fn(0)
        return
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fn, range(n)))


def normal(seed_seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    """Seeded N(0, std^2) float32 draw of ``shape``, chunk-parallel."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    nch = _nchunks(n)
    kids = seed_seq.spawn(nch)

    def work(i):
        g = np.random.Generator(np.random.PCG64(kids[i]))
        s = slice(i * _CHUNK, min(n, (i + 1) * _CHUNK))
        g.standard_normal(out=out[s], dtype=np.float32)
        if std != 1.0:
            out[s] *= np.float32(std)

    _parallel(work, nch)
    return out.reshape(shape)


def zipf_bias(E: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Per-expert logit bias ``-s * ln(rank)`` with ``rank`` a seeded
    permutation of 1..E (the log of an unnormalised Zipf(s) pmf)."""
    rank = rng.permutation(E) + 1
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def uniform_assignment(T: int, k: int, E: int,
                       rng: np.random.Generator) -> np.ndarray:
    """Forced expert ids ``perm[(t*k + j) mod E]`` for slot (t, j).

    The k ids of a token are distinct whenever k <= E, and every expert gets
    exactly T*k/E slots whenever E divides T*k.
    """
    perm = rng.permutation(E).astype(np.int32)
    slots = np.arange(T * k, dtype=np.int64) % E
    return perm[slots].reshape(T, k).astype(np.int32)


def make_inputs(wl: Workload, with_dy: bool = True) -> Inputs:
    """Draw the seeded inputs of ``wl``.

    x, dy ~ N(0, 1); router and expert weights ~ N(0, w_std^2); all drawn in
    float32 and rounded to bf16 for bf16 workloads.
    """
    if not (1 <= wl.k <= wl.E):
        raise ValueError("need 1 <= k <= E")
    root = np.random.SeedSequence(wl.seed)
    s_x, s_wr, s_w1, s_w2, s_dy, s_aux = root.spawn(6)
    x = normal(s_x, (wl.T, wl.d), 1.0)
    wr = normal(s_wr, (wl.d, wl.E), wl.w_std)
    w1 = normal(s_w1, (wl.E, wl.d, 2 * wl.F), wl.w_std)
    w2 = normal(s_w2, (wl.E, wl.F, wl.d), wl.w_std)
    dy = normal(s_dy, (wl.T, wl.d), 1.0) if with_dy else None
    if wl.dtype == "bf16":
        for a in (x, wr, w1, w2, dy):
            if a is not None:
                round_to_bf16(a)
    elif wl.dtype != "fp32":
        raise ValueError(f"unknown dtype {wl.dtype!r}")
    aux = np.random.Generator(np.random.PCG64(s_aux))
    bias = None
    forced = None
    if wl.regime == "skew":
        bias = zipf_bias(wl.E, wl.zipf_s, aux)
    elif wl.regime == "uniform":
        forced = uniform_assignment(wl.T, wl.k, wl.E, aux)
    elif wl.regime != "natural":
        raise ValueError(f"unknown regime {wl.regime!r}")
    return Inputs(wl, x, wr, w1, w2, dy, bias, forced)


def random_topk_ids(T: int, k: int, E: int, seed: int) -> np.ndarray:
    """Seeded expert ids ``[T,k]``: k distinct experts per token, uniform.

    Used to exercise counting/indexing on its own, without a router.
    """
    g = np.random.default_rng(seed)
    keys = g.random((T, E))
    return np.argsort(keys, axis=1)[:, :k].astype(np.int32)


__all__ = ["Workload", "WORKLOADS", "Inputs", "make_inputs", "round_to_bf16",
           "bf16_bits", "normal", "zipf_bias", "uniform_assignment",
           "random_topk_ids"]

