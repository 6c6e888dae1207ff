"""GPU parity of the whole layer (forward + backward through MoELayer, i.e.
through the C ABI, in the launch configuration the benchmark times).

Small shapes: every output compared in full against the oracle.  The five
workload shapes at full size: routing / counts / indices compared in full
(bit-exact), float outputs on sampled tokens and sampled experts that the
oracle computes one by one.  The routing decision is taken on the device's
float32 logits (the oracle's own float64 logits are compared separately), so
near-ties cannot make the two sides route differently."""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import WORKLOADS, Workload, make_inputs
from tests._gpu import (DEV, TOL_BF16, TOL_F32, dev, expert_weight_grads, host, rel,
                        sample_tokens, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _native_lib():
    import mixture_experts_layer_gating_amd._lib  # noqa: F401  (raises if not built)


def _run(inp, renorm=False, fuse_act=True, overlap_wgrad=False):
    from mixture_experts_layer_gating_amd.layer import MoELayer
    wl = inp.wl
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=tdt, device=DEV, renorm=renorm,
                     fuse_act=fuse_act, overlap_wgrad=overlap_wgrad)
    x, wr, w1, w2, dy = (dev(a, tdt) for a in (inp.x, inp.wr, inp.w1, inp.w2, inp.dy))
    bias = None if inp.bias is None else dev(inp.bias)
    forced = None if inp.forced_idx is None else dev(inp.forced_idx)
    layer.forward(x, wr, w1, w2, bias=bias, forced_idx=forced)
    grads = layer.backward(dy)
    torch.cuda.synchronize()
    return layer, grads, (x, wr, w1, w2, dy, bias, forced)


def _full_compare(inp, renorm=False):
    wl = inp.wl
    tol = TOL_BF16 if wl.dtype == "bf16" else TOL_F32
    layer, g, _ = _run(inp, renorm)
    logits = host(layer.logits).astype(np.float32)
    # the device's logits agree with the oracle's own float64 logits
    assert rel(logits, O.router_logits(inp.x, inp.wr)) <= tol
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


@pytest.mark.parametrize("name", FULL)
def test_layer_full_size_sampled(name):
    wl = WORKLOADS[name]
    say(f"layer full size {wl}")
    inp = make_inputs(wl)
    layer, g, _ = _run(inp)
    say("  gpu done")
    k = wl.k
    logits = host(layer.logits).astype(np.float32)
    # routing, counts, indices: full and bit-exact (decision on device logits)
    oidx, ow, op = O.route(logits, k, bias=inp.bias, forced_idx=inp.forced_idx)
    np.testing.assert_array_equal(host(layer.idx), oidx)
    assert rel(host(layer.w), ow) <= TOL_F32
    counts, offsets, dest, src = O.build_index(oidx, wl.E)
    for key, want in (("counts", counts), ("offsets", offsets), ("dest", dest), ("src", src)):
        np.testing.assert_array_equal(host(getattr(layer, key)), want, err_msg=key)
    if wl.regime == "uniform":
        assert (counts == wl.Tk // wl.E).all()
    say(f"  routing ok; rows/expert min {counts.min()} max {counts.max()}")
    # logits of sampled tokens against the oracle's float64 logits
    rng = np.random.default_rng(wl.seed)
    tok = np.sort(rng.choice(wl.T, size=min(64, wl.T), replace=False))
    assert rel(logits[tok], O.router_logits(inp.x[tok], inp.wr)) <= TOL_BF16
    # y, dx, dlogits of sampled tokens
    fwd, bwd = sample_tokens(inp, logits, k, tok)
    tsel = torch.from_numpy(tok).to(DEV)
    errs = {"y": rel(host(layer.y[tsel]), fwd["y"]), "dx": rel(host(g.dx[tsel]), bwd["dx"]),
            "dlogits": rel(host(layer.dlogits[tsel]), bwd["dz"]),
            "dw_gate": rel(host(layer.dw[tsel]), bwd["dw"])}
    # weight gradients of sampled experts: the hottest, the coldest non-empty, one random
    nz = np.flatnonzero(counts)
    experts = sorted({int(np.argmax(counts)), int(nz[np.argmin(counts[nz])]),
                      int(rng.choice(nz))})
    for e in experts:
        rdw1, rdw2, n = expert_weight_grads(inp, k, oidx, ow, e)
        gw1 = host(g.dw1[e])
        errs[f"dw1_gate[{e}]"] = rel(gw1[:, :wl.F], rdw1[:, :wl.F])
        errs[f"dw1_up[{e}]"] = rel(gw1[:, wl.F:], rdw1[:, wl.F:])
        errs[f"dw2[{e}]"] = rel(host(g.dw2[e]), rdw2)
    # router weight gradient: the product x^T @ dlogits of the device's dlogits
    dl = host(layer.dlogits)
    errs["dwr"] = rel(host(g.dwr), inp.x.astype(np.float64).T @ dl)
    say("  errors", {k2: float("%.3g" % v) for k2, v in errs.items()})
    assert max(errs.values()) <= TOL_BF16, errs
    # empty experts have exactly zero weight gradients
    for e in np.flatnonzero(counts == 0)[:4]:
        assert not host(g.dw2[int(e)]).any()


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
