"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one bug in the CPU oracle -- a dropped term, a wrong sign,
a transposed operand, an off-by-one, an unstable order, swapped halves --
and runs the pins that guard that function.  At least one of them must
fail; with the oracle as written all of them pass.  The mistakes are
planted in the oracle only, never in the HIP path.
"""
import numpy as np
import pytest

import oracle as O
import oracle.moe_oracle as OM
from tests import test_oracle_pins as P

F64 = np.float64


# ----------------------------------------------------------------- mutants
def softmax_wrong_axis(z):
    z = np.asarray(z, F64)
    ez = np.exp(z - z.max())
    return ez / ez.sum(axis=0, keepdims=True)


def topk_ties_to_higher_index(z, k):
    z = np.asarray(z)
    E = z.shape[1]
    rev = z[:, ::-1]
    order = np.argsort(-rev, axis=-1, kind="stable")
    return np.ascontiguousarray((E - 1 - order)[:, :k]).astype(np.int32)


def gate_weights_always_renormalised(p, idx, renorm=False):
    w = np.take_along_axis(np.asarray(p, F64), np.asarray(idx, np.int64), axis=1)
    return w / w.sum(axis=1, keepdims=True)


def build_index_unstable(idx, E):
    flat = np.asarray(idx).reshape(-1)
    counts = OM.count_tokens(idx, E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    src = np.empty(flat.size, dtype=np.int32)
    for e in range(E):
        src[offsets[e]:offsets[e + 1]] = np.flatnonzero(flat == e)[::-1]  # reversed in a group
    dest = np.empty(flat.size, dtype=np.int32)
    dest[src] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, dest, src


def build_index_inclusive_offsets(idx, E):
    counts, offsets, dest, src = OM.__dict__["_orig_build_index"](idx, E)
    off = offsets.copy()
    off[:-1] = offsets[1:]  # inclusive instead of exclusive scan
    return counts, off, dest, src


def silu_wrong_sign(z):
    z = np.asarray(z, F64)
    return z * OM.sigmoid(-z)


def swiglu_swapped_halves(h):
    h = np.asarray(h, F64)
    F = h.shape[1] // 2
    return OM.silu(h[:, F:]) * h[:, :F]


def grouped_matmul_transposed(a, w, offsets):
    a = np.asarray(a, F64)
    E, K, N = w.shape
    c = np.zeros((a.shape[0], N), dtype=F64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            we = np.asarray(w[e], F64).reshape(N, K).T  # reads the weights in the wrong order
            c[r0:r1] = a[r0:r1] @ we
    return c


def combine_unweighted(yp, dest, w, k):
    return OM.__dict__["_orig_combine"](yp, dest, np.ones_like(np.asarray(w, F64)), k)


def swiglu_backward_dropped_term(h, da):
    h = np.asarray(h, F64)
    da = np.asarray(da, F64)
    F = h.shape[1] // 2
    g, u = h[:, :F], h[:, F:]
    s = OM.sigmoid(g)
    return np.concatenate([da * u * s, da * g * s], axis=1)  # (1 + g(1 - s)) dropped


def gate_backward_sign(p, idx, dw, renorm=False):
    return -OM.__dict__["_orig_gate_backward"](p, idx, dw, renorm)


def grouped_matmul_backward_no_transpose(a, w, dc, offsets):
    da, dw = OM.__dict__["_orig_grouped_matmul_backward"](a, w, dc, offsets)
    E, K, N = w.shape
    a = np.asarray(a, F64)
    dc = np.asarray(dc, F64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            we = np.asarray(w[e], F64)
            da[r0:r1] = dc[r0:r1] @ we.reshape(N, K)  # w[e] reshaped, not transposed
    return da, dw


def router_backward_no_dx(x, wr, dz):
    dx, dwr = OM.__dict__["_orig_router_backward"](x, wr, dz)
    return np.zeros_like(dx), dwr


def permute_backward_first_slot_only(dxp, dest, k, T):
    dxp = np.asarray(dxp, F64)
    d2 = np.asarray(dest).reshape(T, k)
    return dxp[d2[:, 0]].copy()


def biased_logits_ignores_bias(logits, bias):
    return np.asarray(logits)


def permute_slot_modulo(x, src, k):
    # token of slot s taken as s % k (the slot's position j) instead of s // k
    return np.asarray(x)[np.asarray(src) % k]


def sigmoid_wrong_sign(z):
    z = np.asarray(z, F64)
    return 1.0 / (1.0 + np.exp(z))


def count_tokens_shifted(idx, E):
    flat = np.asarray(idx).reshape(-1)
    return np.array([np.count_nonzero(flat == e + 1) for e in range(E)], dtype=np.int32)


def grouped_matmul_drops_last_row(a, w, offsets):
    a = np.asarray(a, F64)
    E, K, N = w.shape
    c = np.zeros((a.shape[0], N), dtype=F64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1]) - 1
        if r1 > r0:
            c[r0:r1] = a[r0:r1] @ np.asarray(w[e], F64)
    return c


def combine_backward_unscaled(dy, yp, dest, w, k):
    dyp, dw = OM._orig_combine_backward(dy, yp, dest, w, k)
    T = np.asarray(dy).shape[0]
    d2 = np.asarray(dest).reshape(T, k)
    for j in range(k):
        dyp[d2[:, j]] = np.asarray(dy, F64)  # the gate weight left out
    return dyp, dw


def combine_backward_wrong_slot(dy, yp, dest, w, k):
    dyp, dw = OM._orig_combine_backward(dy, yp, dest, w, k)
    dy = np.asarray(dy, F64)
    yp = np.asarray(yp, F64)
    T = dy.shape[0]
    d2 = np.asarray(dest).reshape(T, k)
    for j in range(k):  # dw of slot j from the row of slot j + 1
        dw[:, j] = np.sum(dy * yp[d2[:, (j + 1) % k]], axis=1)
    return dyp, dw


def gate_backward_renorm_term_dropped(p, idx, dw, renorm=False):
    if not renorm:
        return OM._orig_gate_backward(p, idx, dw)
    p = np.asarray(p, F64)
    idx = np.asarray(idx, np.int64)
    S = np.take_along_axis(p, idx, axis=1).sum(axis=1, keepdims=True)
    return OM._orig_gate_backward(p, idx, np.asarray(dw, F64) / S)


# ----------------------------------------------------------------- pins to run
FD = [lambda: P.test_backward_matches_central_differences(False, False, False),
      lambda: P.test_backward_matches_central_differences(True, False, False),
      P.test_adjoint_identities]
DENSE = [lambda: P.test_layer_forward_equals_dense_masked_evaluation(4, 2, False, False),
         lambda: P.test_layer_forward_equals_dense_masked_evaluation(5, 3, True, False),
         P.test_layer_single_expert_is_plain_swiglu_ffn]

CASES = {
    "softmax over the wrong axis": ("softmax", softmax_wrong_axis,
                                    [P.test_softmax_known_values_and_invariants]),
    "top-k ties to the higher index": ("topk_experts", topk_ties_to_higher_index,
                                       [lambda: P.test_topk_matches_brute_force_with_ties(8, 2),
                                        P.test_topk_hand_examples]),
    "gate weights always renormalised": ("gate_weights", gate_weights_always_renormalised,
                                         [P.test_route_weights_closed_forms] + DENSE),
    "unstable order inside a group": ("build_index", build_index_unstable,
                                      [lambda: P.test_counts_and_index_against_library_and_brute_force(64, 8, 64),
                                       P.test_index_hand_example]),
    "inclusive offsets": ("build_index", build_index_inclusive_offsets,
                          [lambda: P.test_counts_and_index_against_library_and_brute_force(7, 2, 3),
                           P.test_index_hand_example]),
    "silu with the wrong sign": ("silu", silu_wrong_sign, [P.test_silu_closed_forms]),
    "swiglu halves swapped": ("swiglu", swiglu_swapped_halves, [P.test_swiglu_hand_example] + DENSE),
    "grouped matmul reads w transposed": ("grouped_matmul", grouped_matmul_transposed,
                                          [P.test_grouped_matmul_brute_force] + DENSE),
    "combine drops the gate weights": ("combine", combine_unweighted, DENSE),
    "swiglu backward drops a term": ("swiglu_backward", swiglu_backward_dropped_term,
                                     [P.test_swiglu_backward_matches_central_differences] + FD),
    "gate backward sign": ("gate_backward", gate_backward_sign,
                           [P.test_gate_backward_matches_central_differences] + FD),
    "grouped matmul backward not transposed": ("grouped_matmul_backward",
                                               grouped_matmul_backward_no_transpose, FD),
    "router backward drops dx": ("router_backward", router_backward_no_dx, FD),
    "permute backward sums one slot": ("permute_backward", permute_backward_first_slot_only, FD),
    "bias left out of the selection scores": ("biased_logits", biased_logits_ignores_bias,
                                              [P.test_route_bias_and_forced,
                                               P.test_biased_logits_add_in_logit_precision]),
    "permute takes the slot's position as its token": ("permute", permute_slot_modulo,
                                                       [P.test_permute_groups_hold_the_routed_tokens]
                                                       + DENSE),
    "sigmoid with the wrong sign": ("sigmoid", sigmoid_wrong_sign, [P.test_silu_closed_forms]),
    "counts shifted by one expert": ("count_tokens", count_tokens_shifted,
                                     [lambda: P.test_counts_and_index_against_library_and_brute_force(64, 8, 64),
                                      P.test_index_hand_example]),
    "grouped matmul drops each group's last row": ("grouped_matmul", grouped_matmul_drops_last_row,
                                                   [P.test_grouped_matmul_brute_force] + DENSE),
    "combine backward leaves out the gate weight": ("combine_backward", combine_backward_unscaled,
                                                    FD),
    "combine backward reads the wrong slot's row": ("combine_backward",
                                                    combine_backward_wrong_slot, FD),
    "gate backward drops the renormalisation term": ("gate_backward",
                                                     gate_backward_renorm_term_dropped,
                                                     [P.test_gate_backward_matches_central_differences]
                                                     + FD),
}


def _plant(monkeypatch, name, fn):
    # keep the original reachable for mutants that wrap it
    monkeypatch.setitem(OM.__dict__, "_orig_" + name, getattr(OM, name))
    monkeypatch.setattr(OM, name, fn)
    monkeypatch.setattr(O, name, fn)


def _fails(pin):
    # A pin fails by an assertion, or by an error the mutant provokes (a
    # count that no longer matches the rows, say): either way it does not pass.
    try:
        pin()
    except Exception:  # noqa: BLE001
        return True
    return False


@pytest.mark.parametrize("case", sorted(CASES))
def test_planted_mistake_is_caught(case, monkeypatch):
    name, fn, pins = CASES[case]
    assert not any(_fails(p) for p in pins), "a pin fails on the oracle as written"
    _plant(monkeypatch, name, fn)
    assert any(_fails(p) for p in pins), f"no pin caught: {case}"
