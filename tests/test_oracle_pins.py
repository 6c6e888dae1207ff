"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks an oracle function against something the mathematics fixes
independently: brute force on tiny inputs, a library routine on a special
case, a closed form, an invariant, or central finite differences of the
forward pass.  The pages print no worked numeric example, so none of the pins
is a value from the pages.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
from moe_inputs import Workload, make_inputs, random_topk_ids


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- softmax
def test_softmax_two_experts_is_logistic():
    # For two experts, p0 = 1 / (1 + exp(z1 - z0)).
    z = np.array([[0.3, -1.1], [5.0, 5.0], [-2.0, 7.5]])
    p = O.softmax(z)
    for row, (z0, z1) in zip(p, z):
        assert row[0] == pytest.approx(1.0 / (1.0 + math.exp(z1 - z0)), rel=1e-15)
        assert row[1] == pytest.approx(1.0 / (1.0 + math.exp(z0 - z1)), rel=1e-15)


def test_softmax_known_values_and_invariants():
    # softmax([0, ln 3]) = [1/4, 3/4]; rows sum to 1; shift invariance.
    p = O.softmax(np.array([[0.0, math.log(3.0)]]))
    assert p[0, 0] == pytest.approx(0.25, rel=1e-15)
    assert p[0, 1] == pytest.approx(0.75, rel=1e-15)
    z = _rng(0).normal(size=(17, 9)) * 10
    p = O.softmax(z)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.softmax(z + 123.0), p, rtol=1e-12, atol=0)
    assert (p > 0).all()


# ----------------------------------------------------------------- top-k
def _brute_topk(z, k):
    out = []
    for row in z:
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
        out.append(order[:k])
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("E,k", [(1, 1), (3, 2), (8, 2), (8, 8), (64, 8), (13, 5)])
def test_topk_matches_brute_force_with_ties(E, k):
    g = _rng(E * 100 + k)
    # Values from a tiny set force many ties.
    z = g.integers(-3, 4, size=(50, E)).astype(np.float32)
    np.testing.assert_array_equal(O.topk_experts(z, k), _brute_topk(z, k))
    z = g.normal(size=(50, E)).astype(np.float32)
    np.testing.assert_array_equal(O.topk_experts(z, k), _brute_topk(z, k))


def test_topk_hand_examples():
    # All equal -> lowest indices first; strictly ordered -> descending.
    z = np.array([[1.0, 1.0, 1.0, 1.0],
                  [0.1, 0.4, 0.3, 0.2],
                  [-0.0, 0.0, -1.0, 2.0]], dtype=np.float32)
    np.testing.assert_array_equal(
        O.topk_experts(z, 2), [[0, 1], [1, 2], [3, 0]])


def test_route_weights_closed_forms():
    g = _rng(3)
    L = g.normal(size=(20, 6))
    # k = E, no renormalisation: every probability is selected, sum is 1.
    idx, w, p = O.route(L, 6)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-14)
    assert sorted(idx[0].tolist()) == list(range(6))
    # Weights are non-increasing in j and equal the softmax probabilities.
    idx, w, p = O.route(L, 3)
    assert (np.diff(w, axis=1) <= 0).all()
    for t in range(20):
        ez = np.exp(L[t] - L[t].max())
        for j in range(3):
            assert w[t, j] == pytest.approx(ez[idx[t, j]] / ez.sum(), rel=1e-13)
    # Renormalised weights sum to one.
    _, wn, _ = O.route(L, 3, renorm=True)
    np.testing.assert_allclose(wn.sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(wn, w / w.sum(axis=1, keepdims=True), rtol=1e-14)


def test_route_bias_and_forced():
    L = np.array([[0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    bias = np.array([-1.0, 0.5, 2.0, 0.5], dtype=np.float32)
    idx, w, p = O.route(L, 2, bias=bias)
    np.testing.assert_array_equal(idx, [[2, 1]])   # tie 1 vs 3 -> 1
    ez = np.exp(bias.astype(np.float64))
    assert w[0, 0] == pytest.approx(ez[2] / ez.sum(), rel=1e-13)
    forced = np.array([[3, 0]], dtype=np.int32)
    idx, w, p = O.route(L, 2, bias=bias, forced_idx=forced)
    np.testing.assert_array_equal(idx, forced)
    assert w[0, 1] == pytest.approx(ez[0] / ez.sum(), rel=1e-13)


def test_biased_logits_add_in_logit_precision():
    # A float32 logit plus a float32 bias is rounded to float32 (R2).
    L = np.array([[1.0, 1.0 + 2 ** -23]], dtype=np.float32)
    b = np.array([2 ** -24, 0.0], dtype=np.float32)
    z = O.biased_logits(L, b)
    assert z.dtype == np.float32
    assert float(z[0, 0]) == 1.0  # 1 + 2^-24 rounds to even -> 1.0


# ----------------------------------------------------------------- counting and indices
@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (7, 2, 3), (64, 8, 64), (513, 2, 8),
                                   (100, 8, 256), (33, 4, 4)])
def test_counts_and_index_against_library_and_brute_force(T, k, E):
    idx = random_topk_ids(T, k, E, seed=T * 7 + E)
    counts, offsets, dest, src = O.build_index(idx, E)
    flat = idx.reshape(-1)
    # Counts: library histogram; total is T*k.
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    assert counts.sum() == T * k
    # Offsets: exclusive prefix sum, built by a plain loop.
    acc = [0]
    for c in counts:
        acc.append(acc[-1] + int(c))
    np.testing.assert_array_equal(offsets, acc)
    # src: the stable sort of the flat expert ids.
    np.testing.assert_array_equal(src, np.argsort(flat, kind="stable"))
    # dest is a bijection onto [0, T*k) and the inverse of src.
    assert sorted(dest.tolist()) == list(range(T * k))
    np.testing.assert_array_equal(src[dest], np.arange(T * k))
    np.testing.assert_array_equal(dest[src], np.arange(T * k))
    # Every slot lands inside its expert's rows.
    for s in range(T * k):
        e = flat[s]
        assert offsets[e] <= dest[s] < offsets[e + 1]


def test_index_hand_example():
    # T=3, k=2, E=3.  Slots (flat s = t*k + j): ids 2,0 | 0,1 | 2,1.
    idx = np.array([[2, 0], [0, 1], [2, 1]], dtype=np.int32)
    counts, offsets, dest, src = O.build_index(idx, 3)
    # Expert 0 holds slots 1, 2; expert 1 holds 3, 5; expert 2 holds 0, 4.
    np.testing.assert_array_equal(counts, [2, 2, 2])
    np.testing.assert_array_equal(offsets, [0, 2, 4, 6])
    np.testing.assert_array_equal(src, [1, 2, 3, 5, 0, 4])
    np.testing.assert_array_equal(dest, [4, 0, 1, 2, 5, 3])


def test_index_all_on_one_expert_and_empty_experts():
    idx = np.full((9, 1), 3, dtype=np.int32)
    counts, offsets, dest, src = O.build_index(idx, 5)
    np.testing.assert_array_equal(counts, [0, 0, 0, 9, 0])
    np.testing.assert_array_equal(offsets, [0, 0, 0, 0, 9, 9])
    np.testing.assert_array_equal(src, np.arange(9))


def test_permute_groups_hold_the_routed_tokens():
    T, k, E, d = 11, 3, 5, 4
    idx = random_topk_ids(T, k, E, seed=5)
    x = _rng(5).normal(size=(T, d))
    counts, offsets, dest, src = O.build_index(idx, E)
    xp = O.permute(x, src, k)
    # Build each expert's rows by walking tokens and slots in order.
    groups = {e: [] for e in range(E)}
    for t in range(T):
        for j in range(k):
            groups[int(idx[t, j])].append(x[t])
    for e in range(E):
        got = xp[offsets[e]:offsets[e + 1]]
        want = np.array(groups[e]).reshape(-1, d)
        np.testing.assert_array_equal(got, want)


# ----------------------------------------------------------------- activation
def test_silu_closed_forms():
    assert O.silu(np.array(0.0)) == 0.0
    assert float(O.silu(np.array(1.0))) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert float(O.silu(np.array(-1.0))) == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert float(O.silu(np.array(40.0))) == pytest.approx(40.0, rel=1e-15)
    assert float(O.silu(np.array(-40.0))) == pytest.approx(-40.0 * math.exp(-40.0), rel=1e-12)
    assert float(O.silu(np.array(-800.0))) == 0.0  # no overflow
    assert float(O.sigmoid(np.array(0.0))) == 0.5


def test_swiglu_hand_example():
    # F = 1: G = 1, U = 2 -> silu(1) * 2 ; G = -2, U = 0.5 -> silu(-2) * 0.5.
    h = np.array([[1.0, 2.0], [-2.0, 0.5]])
    a = O.swiglu(h)
    assert a[0, 0] == pytest.approx(2.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert a[1, 0] == pytest.approx(0.5 * -2.0 / (1.0 + math.exp(2.0)), rel=1e-15)


# ----------------------------------------------------------------- grouped matmul
def test_grouped_matmul_brute_force():
    g = _rng(11)
    E, K, N = 3, 4, 5
    counts = [2, 0, 3]
    offsets = np.array([0, 2, 2, 5])
    a = g.normal(size=(5, K))
    w = g.normal(size=(E, K, N))
    c = O.grouped_matmul(a, w, offsets)
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            for n in range(N):
                s = 0.0
                for kk in range(K):
                    s += a[r, kk] * w[e, kk, n]
                assert c[r, n] == pytest.approx(s, rel=1e-13, abs=1e-15)
    assert sum(counts) == 5


def test_grouped_matmul_uniform_is_batched_matmul():
    g = _rng(12)
    E, m, K, N = 4, 6, 7, 3
    a = g.normal(size=(E * m, K))
    w = g.normal(size=(E, K, N))
    offsets = np.arange(E + 1) * m
    c = O.grouped_matmul(a, w, offsets)
    np.testing.assert_allclose(c, np.matmul(a.reshape(E, m, K), w).reshape(E * m, N),
                               rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------- whole layer, forward
def _tiny(T=9, d=8, E=4, k=2, F=5, seed=0, **kw):
    wl = Workload("t", T=T, d=d, E=E, k=k, F=F, dtype="fp32", w_std=0.5,
                  seed=seed, **kw)
    return make_inputs(wl)


def _dense_reference(x, wr, w1, w2, k, bias=None, renorm=False):
    """Every expert applied to every token, masked by the top-k gate."""
    x = np.asarray(x, np.float64)
    L = x @ np.asarray(wr, np.float64)
    if bias is not None:
        L = L + bias
    E = w1.shape[0]
    F = w1.shape[2] // 2
    G = np.zeros_like(L)
    for t in range(L.shape[0]):
        order = sorted(range(E), key=lambda e: (-L[t, e], e))[:k]
        ez = np.exp(L[t] - L[t].max())
        pr = ez / ez.sum()
        tot = sum(pr[e] for e in order)
        for e in order:
            G[t, e] = pr[e] / tot if renorm else pr[e]
    y = np.zeros_like(x)
    for e in range(E):
        H = x @ np.asarray(w1[e], np.float64)
        gate, up = H[:, :F], H[:, F:]
        act = gate / (1.0 + np.exp(-gate)) * up
        y += G[:, e:e + 1] * (act @ np.asarray(w2[e], np.float64))
    return y


@pytest.mark.parametrize("E,k,renorm,skew", [(4, 2, False, False), (4, 4, False, False),
                                             (5, 3, True, False), (6, 2, False, True),
                                             (8, 1, False, False)])
def test_layer_forward_equals_dense_masked_evaluation(E, k, renorm, skew):
    inp = _tiny(T=13, E=E, k=k, seed=E + k)
    bias = np.linspace(-1, 1, E).astype(np.float32) if skew else None
    fwd = O.layer_forward(inp.x, inp.wr, inp.w1, inp.w2, k, bias=bias, renorm=renorm)
    ref = _dense_reference(inp.x, inp.wr, inp.w1, inp.w2, k, bias=bias, renorm=renorm)
    np.testing.assert_allclose(fwd["y"], ref, rtol=1e-12, atol=1e-13)


def test_layer_single_expert_is_plain_swiglu_ffn():
    # E = 1, k = 1: the gate weight is exactly 1 and y = FFN(x).
    inp = _tiny(T=7, E=1, k=1, seed=21)
    fwd = O.layer_forward(inp.x, inp.wr, inp.w1, inp.w2, 1)
    assert (fwd["w"] == 1.0).all()
    x = inp.x.astype(np.float64)
    H = x @ inp.w1[0].astype(np.float64)
    F = H.shape[1] // 2
    want = (H[:, :F] / (1 + np.exp(-H[:, :F])) * H[:, F:]) @ inp.w2[0].astype(np.float64)
    np.testing.assert_allclose(fwd["y"], want, rtol=1e-12, atol=1e-14)


def test_layer_forced_uniform_counts():
    wl = Workload("u", T=32, d=8, E=8, k=2, F=4, dtype="fp32", seed=4, regime="uniform")
    inp = make_inputs(wl)
    fwd = O.layer_forward(inp.x, inp.wr, inp.w1, inp.w2, 2, forced_idx=inp.forced_idx)
    np.testing.assert_array_equal(fwd["counts"], np.full(8, 8))
    ref_idx = inp.forced_idx
    np.testing.assert_array_equal(fwd["idx"], ref_idx)


# ----------------------------------------------------------------- backward
def _loss(inp, k, dy, bias=None, renorm=False, forced=None, **over):
    x = over.get("x", inp.x)
    wr = over.get("wr", inp.wr)
    w1 = over.get("w1", inp.w1)
    w2 = over.get("w2", inp.w2)
    f = O.layer_forward(x, wr, w1, w2, k, bias=bias, forced_idx=forced, renorm=renorm)
    return float(np.sum(f["y"] * dy)), f["idx"]


@pytest.mark.parametrize("renorm,skew,forced", [(False, False, False), (True, False, False),
                                                (False, True, False), (False, False, True)])
def test_backward_matches_central_differences(renorm, skew, forced):
    T, d, E, k, F = 6, 8, 4, 2, 5
    wl = Workload("fd", T=T, d=d, E=E, k=k, F=F, dtype="fp32", w_std=0.5, seed=31,
                  regime="uniform" if forced else "natural")
    inp = make_inputs(wl)
    for name in ("x", "wr", "w1", "w2"):
        setattr(inp, name, getattr(inp, name).astype(np.float64))
    bias = np.array([0.3, -0.2, 0.1, 0.0]) if skew else None
    fidx = inp.forced_idx if forced else None
    dy = inp.dy.astype(np.float64)
    fwd = O.layer_forward(inp.x, inp.wr, inp.w1, inp.w2, k, bias=bias, forced_idx=fidx,
                          renorm=renorm)
    bwd = O.layer_backward(fwd, dy, inp.x, inp.wr, inp.w1, inp.w2, k, renorm=renorm)
    g = _rng(99)
    h = 1e-6
    checked = 0
    for name, grad in (("x", bwd["dx"]), ("wr", bwd["dwr"]), ("w1", bwd["dw1"]),
                       ("w2", bwd["dw2"])):
        base = getattr(inp, name)
        for _ in range(12):
            pos = tuple(int(g.integers(0, s)) for s in base.shape)
            plus = base.copy(); plus[pos] += h
            minus = base.copy(); minus[pos] -= h
            lp, ip = _loss(inp, k, dy, bias, renorm, fidx, **{name: plus})
            lm, im = _loss(inp, k, dy, bias, renorm, fidx, **{name: minus})
            if not (np.array_equal(ip, fwd["idx"]) and np.array_equal(im, fwd["idx"])):
                continue  # the step changes the selected set: not differentiable here
            fd = (lp - lm) / (2 * h)
            assert grad[pos] == pytest.approx(fd, rel=1e-6, abs=1e-9), (name, pos)
            checked += 1
    assert checked >= 40


def test_gate_backward_matches_central_differences():
    g = _rng(7)
    T, E, k = 5, 6, 3
    L = g.normal(size=(T, E))
    c = g.normal(size=(T, k))
    for renorm in (False, True):
        idx, w, p = O.route(L, k, renorm=renorm)
        dz = O.gate_backward(p, idx, c, renorm=renorm)
        h = 1e-6
        for t, e in itertools.product(range(T), range(E)):
            Lp = L.copy(); Lp[t, e] += h
            Lm = L.copy(); Lm[t, e] -= h
            fp = np.sum(O.gate_weights(O.softmax(Lp), idx, renorm) * c)
            fm = np.sum(O.gate_weights(O.softmax(Lm), idx, renorm) * c)
            assert dz[t, e] == pytest.approx((fp - fm) / (2 * h), rel=1e-6, abs=1e-9)


def test_swiglu_backward_matches_central_differences():
    g = _rng(8)
    hmat = g.normal(size=(4, 6)) * 3
    da = g.normal(size=(4, 3))
    dh = O.swiglu_backward(hmat, da)
    eps = 1e-6
    for pos in itertools.product(range(4), range(6)):
        hp = hmat.copy(); hp[pos] += eps
        hm = hmat.copy(); hm[pos] -= eps
        fd = (np.sum(O.swiglu(hp) * da) - np.sum(O.swiglu(hm) * da)) / (2 * eps)
        assert dh[pos] == pytest.approx(fd, rel=1e-6, abs=1e-10)
    # silu'(0) = 1/2 (closed form): G = 0, U = 1.
    assert O.swiglu_backward(np.array([[0.0, 1.0]]), np.array([[1.0]]))[0, 0] == 0.5


def test_adjoint_identities():
    g = _rng(9)
    T, k, E, d = 10, 3, 4, 6
    idx = random_topk_ids(T, k, E, seed=9)
    _, offsets, dest, src = O.build_index(idx, E)
    x = g.normal(size=(T, d))
    v = g.normal(size=(T * k, d))
    # <P x, v> = <x, P^T v> with P = permute and P^T = permute_backward.
    lhs = np.sum(O.permute(x, src, k) * v)
    rhs = np.sum(x * O.permute_backward(v, dest, k, T))
    assert lhs == pytest.approx(rhs, rel=1e-13)
    # combine is bilinear in (yp, w): <C(yp, w), u> = <yp, dyp(u)> = <w, dw(u)>.
    yp = g.normal(size=(T * k, d))
    w = g.random(size=(T, k))
    u = g.normal(size=(T, d))
    dyp, dw = O.combine_backward(u, yp, dest, w, k)
    ref = np.sum(O.combine(yp, dest, w, k) * u)
    assert np.sum(yp * dyp) == pytest.approx(ref, rel=1e-13)
    assert np.sum(w * dw) == pytest.approx(ref, rel=1e-13)
    # grouped matmul: <G(a), c> = <a, da(c)> = <w, dw(c)>.
    K, N = d, 5
    wt = g.normal(size=(E, K, N))
    cc = g.normal(size=(T * k, N))
    da, dwt = O.grouped_matmul_backward(v, wt, cc, offsets)
    ref = np.sum(O.grouped_matmul(v, wt, offsets) * cc)
    assert np.sum(v * da) == pytest.approx(ref, rel=1e-12)
    assert np.sum(wt * dwt) == pytest.approx(ref, rel=1e-12)


def test_empty_expert_gets_zero_weight_gradient():
    idx = np.array([[0, 2], [2, 0], [0, 2]], dtype=np.int32)
    _, offsets, dest, src = O.build_index(idx, 3)
    a = _rng(1).normal(size=(6, 4))
    w = _rng(2).normal(size=(3, 4, 5))
    dc = _rng(3).normal(size=(6, 5))
    _, dw = O.grouped_matmul_backward(a, w, dc, offsets)
    assert (dw[1] == 0).all() and offsets[1] == offsets[2]


def test_rel_fro():
    assert O.rel_fro([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert O.rel_fro([3.0, 4.0 + 0.5], [3.0, 4.0]) == pytest.approx(0.1)
    assert O.rel_fro([0.0], [0.0]) == 0.0
