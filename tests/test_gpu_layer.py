"""GPU parity of the whole layer (forward + backward through MoELayer, i.e.
through the C ABI, in the launch configuration the benchmark times).

Small shapes and the five workload shapes at full size: every output compared
in full against the oracle.  The router logits are held to the oracle's own
float64 logits (1e-5), and routing flips against the oracle's routing on those
logits are counted and must all be near ties; the routing decision compared
bit-exactly is the oracle's on the device's float32 logits (the decision is
taken in the logits' own precision)."""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import WORKLOADS, Workload, make_inputs
from tests._gpu import (DEV, TOL_BF16, TOL_F32, TOL_LOGITS, dev, host, rel, rel_by_expert,
                        routing_flips, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _native_lib():
    import mixture_experts_layer_gating_amd._lib  # noqa: F401  (raises if not built)


def _run(inp, renorm=False, fuse_act=True, overlap_wgrad=False, gather_dy=True):
    from mixture_experts_layer_gating_amd.layer import MoELayer
    wl = inp.wl
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=tdt, device=DEV, renorm=renorm,
                     fuse_act=fuse_act, overlap_wgrad=overlap_wgrad, gather_dy=gather_dy)
    x, wr, w1, w2, dy = (dev(a, tdt) for a in (inp.x, inp.wr, inp.w1, inp.w2, inp.dy))
    bias = None if inp.bias is None else dev(inp.bias)
    forced = None if inp.forced_idx is None else dev(inp.forced_idx)
    layer.forward(x, wr, w1, w2, bias=bias, forced_idx=forced)
    grads = layer.backward(dy)
    torch.cuda.synchronize()
    return layer, grads, (x, wr, w1, w2, dy, bias, forced)


def _full_compare(inp, renorm=False, gather_dy=True):
    wl = inp.wl
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_F32
    layer, g, _ = _run(inp, renorm, gather_dy=gather_dy)
    logits = host(layer.logits).astype(np.float32)
    # the device's logits agree with the oracle's own float64 logits (float32
    # sums of exactly representable products)
    ologits = O.router_logits(inp.x, inp.wr)
    assert rel(logits, ologits) <= TOL_LOGITS
    if inp.forced_idx is None:
        _, bad = routing_flips(host(layer.idx), O.biased_logits(ologits, inp.bias), wl.k)
        assert not bad, f"tokens {bad[:8]} route differently without a near tie"
    fwd = O.layer_forward(inp.x, inp.wr, inp.w1, inp.w2, wl.k, bias=inp.bias,
                          forced_idx=inp.forced_idx, renorm=renorm, logits=logits)
    bwd = O.layer_backward(fwd, inp.dy, inp.x, inp.wr, inp.w1, inp.w2, wl.k, renorm=renorm)
    for key in ("idx", "counts", "offsets", "dest", "src"):
        np.testing.assert_array_equal(host(getattr(layer, key)).reshape(-1),
                                      np.asarray(fwd[key]).reshape(-1), err_msg=key)
    assert rel(host(layer.w), fwd["w"]) <= TOL_F32
    errs = {"y": rel(host(layer.y), fwd["y"]), "dx": rel(host(g.dx), bwd["dx"]),
            "dwr": rel(host(g.dwr), bwd["dwr"]),
            "dw1_gate": rel(host(g.dw1)[:, :, :wl.F], bwd["dw1"][:, :, :wl.F]),
            "dw1_up": rel(host(g.dw1)[:, :, wl.F:], bwd["dw1"][:, :, wl.F:]),
            "dw2": rel(host(g.dw2), bwd["dw2"])}
    say("  errors", {k: float("%.3g" % v) for k, v in errs.items()})
    assert max(errs.values()) <= tol, errs
    return layer


def test_layer_tiny_fp32():
    wl = WORKLOADS["tiny"]
    say(f"layer {wl}")
    _full_compare(make_inputs(wl))


SMALL = [
    dict(T=1024, d=512, E=8, k=2, F=384),     # several tiles, ragged groups
    dict(T=333, d=256, E=16, k=4, F=136),     # ragged everything
    dict(T=64, d=128, E=1, k=1, F=64),        # single expert: plain SwiGLU FFN
    dict(T=256, d=256, E=64, k=8, F=128),     # small groups, empty experts
    dict(T=1, d=64, E=4, k=4, F=32),          # one token, every expert selected (k = E)
    dict(T=37, d=72, E=5, k=1, F=40),         # top-1, widths not multiples of 64
    dict(T=96, d=64, E=1024, k=32, F=32),     # the largest E and k the library takes
]


@pytest.mark.parametrize("shape", SMALL)
def test_layer_small_bf16(shape):
    wl = Workload("small", dtype="bf16", w_std=0.05, seed=sum(shape.values()), **shape)
    say(f"layer {wl}")
    _full_compare(make_inputs(wl))


@pytest.mark.parametrize("shape", [SMALL[0], SMALL[1], SMALL[3]])
def test_layer_written_dyp_bf16(shape):
    """The backward pass with the combine's gradient written (gather_dy=False)
    against the oracle, as the default gathered path is."""
    wl = Workload("dyp", dtype="bf16", w_std=0.05, seed=sum(shape.values()) + 1, **shape)
    say(f"layer written dyp {wl}")
    _full_compare(make_inputs(wl), gather_dy=False)


def test_layer_ragged_fp32():
    # float32 at widths off the MFMA path (FMA kernels throughout)
    wl = Workload("ragged", T=100, d=40, E=6, k=3, F=24, dtype="fp32", w_std=0.05, seed=5)
    say(f"layer {wl}")
    _full_compare(make_inputs(wl))


@pytest.mark.parametrize("regime", ["skew", "uniform"])
@pytest.mark.parametrize("renorm", [False, True])
def test_layer_regimes_bf16(regime, renorm):
    wl = Workload("regime", T=1024, d=256, E=16, k=4, F=128, dtype="bf16", w_std=0.05,
                  seed=3, regime=regime)
    say(f"layer {wl} renorm={renorm}")
    layer = _full_compare(make_inputs(wl), renorm=renorm)
    if regime == "uniform":
        assert (host(layer.counts) == wl.Tk // wl.E).all()


def test_layer_deterministic():
    wl = Workload("det", T=2048, d=512, E=16, k=4, F=256, dtype="bf16", w_std=0.05, seed=11)
    say("layer determinism")
    inp = make_inputs(wl)
    l1, g1, _ = _run(inp)
    snap = [t.clone() for t in (l1.idx, l1.dest, l1.y, g1.dx, g1.dwr, g1.dw1, g1.dw2)]
    l2, g2, _ = _run(inp)
    for a, b in zip(snap, (l2.idx, l2.dest, l2.y, g2.dx, g2.dwr, g2.dw1, g2.dw2)):
        assert torch.equal(a, b)


def test_layer_graph_replay():
    """The step captured as a HIP graph: every replay gives the bits of an
    eager step on the same inputs, also after the inputs are rewritten in
    place and with eager steps between replays."""
    from mixture_experts_layer_gating_amd.layer import MoELayer
    wl = Workload("graph", T=1024, d=512, E=16, k=4, F=256, dtype="bf16", w_std=0.05, seed=21)
    say("layer graph capture and replay")
    bf = torch.bfloat16
    inp_a = make_inputs(wl)
    inp_b = make_inputs(wl.with_(seed=22))
    a = [dev(t, bf) for t in (inp_a.x, inp_a.wr, inp_a.w1, inp_a.w2, inp_a.dy)]
    b = [dev(t, bf) for t in (inp_b.x, inp_b.wr, inp_b.w1, inp_b.w2, inp_b.dy)]
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=bf, device=DEV)

    def outs():
        g = Grads_of(layer)
        return [t.clone() for t in (layer.idx, layer.dest, layer.y) + g]

    def Grads_of(lay):
        return (lay.dx, lay.dwr, lay.dw1, lay.dw2)

    def eager(inp):
        layer.forward(*inp[:4])
        layer.backward(inp[4])
        torch.cuda.synchronize()
        return outs()

    want_a, want_b = eager(a), eager(b)
    bufs = [t.clone() for t in a]
    graph = layer.capture(*bufs)
    for want, src in ((want_a, a), (want_b, b), (want_b, b), (want_a, a)):
        for buf, t in zip(bufs, src):
            buf.copy_(t)
        graph.replay()
        torch.cuda.synchronize()
        for got, w in zip(outs(), want):
            assert torch.equal(got, w)
        eager(b)  # eager work between replays


# ------------------------------------------------------------------ full-size workloads
FULL = ["olmoe", "olmoe_skew", "olmoe_uniform", "sparse", "large"]


@pytest.mark.parametrize("name", [pytest.param(n, marks=pytest.mark.timeout(900)) for n in FULL])
def test_layer_full_size(name):
    """The five workload shapes at full size, every output compared in full
    against one whole oracle pass:

    * router logits against the oracle's own float64 logits (<= 1e-5);
    * routing flips against the oracle's routing on those float64 logits:
      every token whose ids differ must be a near tie (the device's j-th pick
      holds, in the float64 scores, the j-th largest value within
      1e-5 * max |score| of the token); the count is printed;
    * ids, counts, offsets, dest, src bit-exact against the oracle's routing
      on the device's float32 logits (the decision is taken in the logits'
      own precision), gate weights <= 1e-5;
    * y, dx, dlogits, the gate-weight gradient, dwr, every expert's dW1
      (gate and up halves) and dW2 against the oracle pass routed on those
      logits, <= 1e-2 (bf16 storage, float32 accumulation)."""
    wl = WORKLOADS[name]
    say(f"layer full size {wl}")
    inp = make_inputs(wl)
    layer, g, _ = _run(inp)
    say("  gpu done")
    k, E = wl.k, wl.E
    logits = host(layer.logits).astype(np.float32)
    # logits against the oracle's float64 logits
    ologits = O.router_logits(inp.x, inp.wr)
    errs = {"logits": rel(logits, ologits)}
    assert errs["logits"] <= TOL_LOGITS, errs
    idx = host(layer.idx)
    if inp.forced_idx is None:
        diff, bad = routing_flips(idx, O.biased_logits(ologits, inp.bias), k)
        say(f"  routing flips against float64 logits: {len(diff)} tokens, "
            f"{len(bad)} not near ties")
        assert not bad, f"tokens {bad[:8]} route differently without a near tie"
    else:
        np.testing.assert_array_equal(idx, inp.forced_idx)
    # the whole oracle pass, routed on the device's float32 logits
    fwd = O.layer_forward(inp.x, inp.wr, inp.w1, inp.w2, k, bias=inp.bias,
                          forced_idx=inp.forced_idx, logits=logits)
    say("  oracle forward done")
    for key in ("idx", "counts", "offsets", "dest", "src"):
        np.testing.assert_array_equal(host(getattr(layer, key)).reshape(-1),
                                      np.asarray(fwd[key]).reshape(-1), err_msg=key)
    counts = fwd["counts"]
    if wl.regime == "uniform":
        assert (counts == wl.Tk // E).all()
    say(f"  routing ok; rows/expert min {counts.min()} max {counts.max()}")
    assert rel(host(layer.w), fwd["w"]) <= TOL_F32
    errs["y"] = rel(host(layer.y), fwd["y"])
    bwd = O.layer_backward(fwd, inp.dy, inp.x, inp.wr, inp.w1, inp.w2, k)
    del fwd
    say("  oracle backward done")
    errs.update({"dx": rel(host(g.dx), bwd["dx"]), "dlogits": rel(host(layer.dlogits), bwd["dz"]),
                 "dw_gate": rel(host(layer.dw), bwd["dw"]), "dwr": rel(host(g.dwr), bwd["dwr"]),
                 "dw1_gate": rel_by_expert(g.dw1, bwd["dw1"], slice(0, wl.F)),
                 "dw1_up": rel_by_expert(g.dw1, bwd["dw1"], slice(wl.F, 2 * wl.F)),
                 "dw2": rel_by_expert(g.dw2, bwd["dw2"])})
    say("  errors", {k2: float("%.3g" % v) for k2, v in errs.items()})
    assert max(v for k2, v in errs.items() if k2 != "logits") <= TOL_BF16, errs
    # empty experts have exactly zero weight gradients
    for e in np.flatnonzero(counts == 0):
        assert not host(g.dw1[int(e)]).any() and not host(g.dw2[int(e)]).any()


def test_layer_fused_activation_matches_unfused():
    """GEMM 1 with the SwiGLU epilogue gives the same bits as GEMM 1 followed
    by the activation kernel, through the whole forward and backward."""
    wl = Workload("fuse", T=1024, d=512, E=8, k=2, F=384, dtype="bf16", w_std=0.05, seed=31)
    say(f"layer fused vs unfused {wl}")
    inp = make_inputs(wl)
    la, ga, _ = _run(inp, fuse_act=True)
    ya, ha, aa = (host(t).copy() for t in (la.y, la.h, la.a))
    da = {k: host(getattr(ga, k)).copy() for k in ("dx", "dwr", "dw1", "dw2")}
    lb, gb, _ = _run(inp, fuse_act=False)
    rows = slice(0, wl.T * wl.k)
    np.testing.assert_array_equal(ha[rows], host(lb.h)[rows])
    np.testing.assert_array_equal(aa[rows], host(lb.a)[rows])
    np.testing.assert_array_equal(ya, host(lb.y))
    for k, v in da.items():
        np.testing.assert_array_equal(v, host(getattr(gb, k)), err_msg=k)


@pytest.mark.parametrize("mode", ["act", "layer"])
def test_layer_recompute_modes_match(mode):
    """Selective recomputation: with recompute="act" the backward pass
    recomputes the SwiGLU output from h, with "layer" it re-runs the whole
    forward from the inputs.  Everything the mode does not keep is overwritten
    with garbage between the passes, and the gradients must still be the bits
    of the keep-everything layer."""
    from mixture_experts_layer_gating_amd.layer import MoELayer
    wl = Workload("recompute", T=1024, d=512, E=16, k=4, F=256, dtype="bf16", w_std=0.05,
                  seed=43, regime="skew")
    say(f"layer recompute={mode} {wl}")
    inp = make_inputs(wl)
    la, ga, args = _run(inp)
    want = {n: host(getattr(ga, n)).copy() for n in ("dx", "dwr", "dw1", "dw2")}
    want["y"] = host(la.y).copy()
    x, wr, w1, w2, dy, bias, forced = args
    lb = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=torch.bfloat16, device=DEV,
                  recompute=mode)
    for _ in range(2):
        lb.forward(x, wr, w1, w2, bias=bias, forced_idx=forced)
        lost = ["a"] if mode == "act" else ["logits", "probs", "idx", "w", "counts", "offsets",
                                            "dest", "src", "h", "a", "yp", "y"]
        for n in lost:
            t = getattr(lb, n)
            if t.dtype == torch.int32:
                t.fill_(7)   # a valid but wrong row/expert everywhere
            else:
                t.fill_(float("nan"))
        gb = lb.backward(dy)
        torch.cuda.synchronize()
        for n in ("dx", "dwr", "dw1", "dw2"):
            np.testing.assert_array_equal(host(getattr(gb, n)), want[n], err_msg=n)
        if mode == "layer":
            np.testing.assert_array_equal(host(lb.y), want["y"])
    kept = lb.saved_bytes()
    full = lb.saved_bytes("none")
    # with dy read through the row map (the default) the backward never reads
    # `a`, so "none" already leaves it out
    assert (kept == {}) if mode == "layer" else (kept == full and "a" not in kept)


def test_layer_overlapped_weight_gradients_match():
    """The weight-gradient GEMMs on a second stream give the same bits as the
    one-stream sequence, over two steps in a row (the second step's forward
    must not overwrite what the first step's side stream still reads)."""
    wl = Workload("ovl", T=2048, d=512, E=16, k=4, F=256, dtype="bf16", w_std=0.05, seed=37,
                  regime="skew")
    say(f"layer overlapped weight gradients {wl}")
    inp = make_inputs(wl)
    la, ga, args = _run(inp, overlap_wgrad=False)
    want = {k: host(getattr(ga, k)).copy() for k in ("dx", "dwr", "dw1", "dw2")}
    lb, gb, _ = _run(inp, overlap_wgrad=True)
    x, wr, w1, w2, dy, bias, forced = args
    for _ in range(2):
        for k, v in want.items():
            np.testing.assert_array_equal(v, host(getattr(gb, k)), err_msg=k)
        lb.forward(x, wr, w1, w2, bias=bias, forced_idx=forced)
        gb = lb.backward(dy)
        torch.cuda.synchronize()
