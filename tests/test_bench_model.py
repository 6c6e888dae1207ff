"""The benchmark's work model (algorithmic FLOPs and bytes per call) against
the closed forms of the layer: the roofline figures divide by these."""
import pytest

import bench
from moe_inputs import WORKLOADS

EXPERT_GEMMS = ("gemm1_swiglu_fwd", "gemm2_fwd", "gemm2_bwd_da", "gemm2_bwd_dw",
                "gemm1_bwd_da", "gemm1_bwd_dw")


@pytest.mark.parametrize("name", ["tiny", "olmoe", "large", "sparse"])
def test_expert_and_router_flops(name):
    wl = WORKLOADS[name]
    b = 2 if wl.dtype == "bf16" else 4
    w = bench.call_work(wl, b)
    Tk, d, F, T, E = wl.T * wl.k, wl.d, wl.F, wl.T, wl.E
    # forward 2 Tk d 2F + 2 Tk F d, backward twice that: 18 Tk d F in all
    assert sum(w[n][0] for n in EXPERT_GEMMS) == 18 * Tk * d * F
    # router: forward 2 T d E, backward 4 T d E
    assert sum(w[n][0] for n in ("router_fwd", "router_bwd_da", "router_bwd_dw")) == 6 * T * d * E
    assert tuple(bench.EXPERT_GEMMS) == EXPERT_GEMMS


def test_olmoe_figures():
    wl = WORKLOADS["olmoe"]
    w = bench.call_work(wl, 2)
    assert abs(sum(w[n][0] for n in EXPERT_GEMMS) / 1e12 - 2.474) < 1e-3  # TFLOP per step
    # permutation: read x once, write Tk rows, read the int32 row map
    assert w["permute"][1] == wl.T * wl.d * 2 + wl.T * wl.k * wl.d * 2 + wl.T * wl.k * 4
    # combine: read Tk rows, write T rows, read dest and w
    assert w["unpermute"][1] == wl.T * wl.k * wl.d * 2 + wl.T * wl.d * 2 + wl.T * wl.k * 8
    # the dominant (NT) calls sit above the ridge point, the small-group ones below
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    for n in ("gemm1_bwd_da", "gemm2_bwd_da"):
        assert w[n][0] / w[n][1] > ridge
    ws = bench.call_work(WORKLOADS["sparse"], 2)
    for n in EXPERT_GEMMS:
        assert ws[n][0] / ws[n][1] < ridge
