"""The oracle's precision switch (float32 for the CPU throughput baseline):
same definitions in another dtype, so its results agree with the float64
oracle to float32 rounding, and the switch restores float64 on exit."""
import numpy as np

import oracle as O
from oracle import moe_oracle as OM
from moe_inputs import Workload, make_inputs


def test_float32_mode_matches_float64():
    wl = Workload("prec", T=96, d=64, E=8, k=2, F=48, dtype="bf16", w_std=0.05, seed=4,
                  regime="skew")
    inp = make_inputs(wl)
    f64 = O.layer_forward(inp.x, inp.wr, inp.w1, inp.w2, wl.k, bias=inp.bias)
    b64 = O.layer_backward(f64, inp.dy, inp.x, inp.wr, inp.w1, inp.w2, wl.k)
    with O.precision(np.float32):
        assert OM.FT is np.float32
        f32 = O.layer_forward(inp.x, inp.wr, inp.w1, inp.w2, wl.k, bias=inp.bias,
                              logits=f64["logits"])
        b32 = O.layer_backward(f32, inp.dy, inp.x, inp.wr, inp.w1, inp.w2, wl.k)
    assert OM.FT is np.float64
    assert f32["y"].dtype == np.float32 and b32["dw1"].dtype == np.float32
    np.testing.assert_array_equal(f32["idx"], f64["idx"])
    assert O.rel_fro(f32["y"], f64["y"]) < 1e-5
    for key in ("dx", "dwr", "dw1", "dw2"):
        assert O.rel_fro(b32[key], b64[key]) < 1e-5, key


def test_precision_restored_after_error():
    try:
        with O.precision(np.float32):
            raise KeyError("x")
    except KeyError:
        pass
    assert OM.FT is np.float64
