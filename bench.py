#!/usr/bin/env python
"""Benchmark: one forward+backward step of the sparse MoE layer on one MI355X.

Workload (default ``olmoe``): T = 8192 tokens (4 x 2048), d = 2048, E = 64
experts, top-8 softmax gate, SwiGLU experts with d_ff = 1024, bf16 storage with
fp32 accumulation, seeded synthetic inputs resident in HBM before timing.

A step is one pass of the whole path: router GEMM, top-k routing, token
counting / index generation, permutation, grouped GEMM 1, SwiGLU, grouped
GEMM 2, weighted combine, and the backward pass of all of them (dx, dW1, dW2,
d_router).  Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--cpu-tokens N | --no-cpu-baseline] [--copy-probe]

``--copy-probe`` adds a plain 1 GiB device copy (torch ``copy_``) after the
timed region, whose counters calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE layer fwd+bwd tokens/sec and grouped-GEMM % of bf16 MFMA peak, 1 GPU"
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_gating_amd", "csrc", "gemm.hip")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- work model
def call_work(wl, b):
    """Algorithmic FLOPs and HBM bytes of each library call of one step.

    Bytes count each input read once and each output written once (``b`` =
    bytes per activation / weight element; indices and gate values 4 B)."""
    T, d, E, k, F = wl.T, wl.d, wl.E, wl.k, wl.F
    Tk = T * k
    f = {}
    f["router_fwd"] = (2 * T * d * E, T * d * b + d * E * b + T * E * 4)
    f["route_topk"] = (0, T * E * 4 * 2 + Tk * 8)
    f["count_index"] = (0, Tk * 4 * 2 + Tk * 4 * 2 + (E + 1) * 8)
    f["permute"] = (0, T * d * b + Tk * d * b + Tk * 4)
    f["gemm1_fwd"] = (2 * Tk * d * 2 * F, Tk * d * b + E * d * 2 * F * b + Tk * 2 * F * b)
    f["act_fwd"] = (0, Tk * 2 * F * b + Tk * F * b)
    f["gemm2_fwd"] = (2 * Tk * F * d, Tk * F * b + E * F * d * b + Tk * d * b)
    f["unpermute"] = (0, Tk * d * b + T * d * b + Tk * 8)
    f["unpermute_bwd"] = (0, T * d * b + 2 * Tk * d * b + Tk * 12)
    f["gemm2_bwd_da"] = (2 * Tk * d * F, Tk * d * b + E * F * d * b + Tk * F * b)
    f["gemm2_bwd_dw"] = (2 * Tk * F * d, Tk * F * b + Tk * d * b + E * F * d * 4)
    f["act_bwd"] = (0, Tk * 2 * F * b + Tk * F * b + Tk * 2 * F * b)
    f["gemm1_bwd_da"] = (2 * Tk * 2 * F * d, Tk * 2 * F * b + E * d * 2 * F * b + Tk * d * b)
    f["gemm1_bwd_dw"] = (2 * Tk * d * 2 * F, Tk * d * b + Tk * 2 * F * b + E * d * 2 * F * 4)
    f["permute_bwd"] = (0, Tk * d * b + T * d * b + Tk * 4)
    f["route_topk_bwd"] = (0, T * E * 4 + Tk * 8 + T * E * b)
    f["router_bwd_da"] = (2 * T * E * d, T * E * b + d * E * b + 2 * T * d * b)
    f["router_bwd_dw"] = (2 * T * d * E, T * d * b + T * E * b + d * E * 4)
    return f


GEMM_CALLS = {  # call -> (product, M, K, N, E) builder
    "router_fwd": lambda wl: (0, wl.T, wl.d, wl.E, 1),
    "gemm1_fwd": lambda wl: (0, wl.T * wl.k, wl.d, 2 * wl.F, wl.E),
    "gemm2_fwd": lambda wl: (0, wl.T * wl.k, wl.F, wl.d, wl.E),
    "gemm2_bwd_da": lambda wl: (1, wl.T * wl.k, wl.F, wl.d, wl.E),
    "gemm2_bwd_dw": lambda wl: (2, wl.T * wl.k, wl.F, wl.d, wl.E),
    "gemm1_bwd_da": lambda wl: (1, wl.T * wl.k, wl.d, 2 * wl.F, wl.E),
    "gemm1_bwd_dw": lambda wl: (2, wl.T * wl.k, wl.d, 2 * wl.F, wl.E),
    "router_bwd_da": lambda wl: (1, wl.T, wl.d, wl.E, 1),
    "router_bwd_dw": lambda wl: (2, wl.T, wl.d, wl.E, 1),
}
EXPERT_GEMMS = ("gemm1_fwd", "gemm2_fwd", "gemm2_bwd_da", "gemm2_bwd_dw", "gemm1_bwd_da",
                "gemm1_bwd_dw")


def kernel_name(L, call, wl, code):
    """Name (as rocprofv3 prints it) of the kernel a GEMM call launches."""
    prod, M, K, N, E = GEMM_CALLS[call](wl)
    plan = L.moe_grouped_gemm_plan(prod, M, K, N, E, code)
    if not plan["mfma"]:
        return f"gemm_simt_kernel<{prod}, ...>"
    out = "unsigned short" if prod == 1 or (prod == 0 and call != "router_fwd") else "float"
    return f"gemm_mfma_kernel<{prod}, {plan['tile_m']}, {plan['tile_n']}, {out}>"


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(inp, tokens):
    """Time the CPU oracle (float64 NumPy, as it stands) on the first
    ``tokens`` tokens of the same workload: forward + backward."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    cores = max(1, min(16, cores))
    wl = inp.wl
    t = np.arange(tokens)
    with threadpool_limits(limits=cores):
        info = threadpool_info()
        used = max([i.get("num_threads", 1) for i in info] or [1])
        x = inp.x[t]
        t0 = time.perf_counter()
        fwd = O.layer_forward(x, inp.wr, inp.w1, inp.w2, wl.k, bias=inp.bias,
                              forced_idx=None if inp.forced_idx is None else inp.forced_idx[t])
        O.layer_backward(fwd, inp.dy[t], x, inp.wr, inp.w1, inp.w2, wl.k)
        dt = time.perf_counter() - t0
    return {"value": round(tokens / dt, 3), "unit": "tokens/s", "cores": int(used),
            "kind": "oracle",
            "sample": (f"first {tokens} of {wl.T} tokens of the same layer (full weights), "
                       f"float64 NumPy forward+backward, {dt:.1f} s")}


# ---------------------------------------------------------------- traffic
def read_traffic(kernel):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 --pmc
    summary, if that summary was taken on the current grouped-GEMM source."""
    sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    path = os.path.join(PROFILES, "gemm_traffic_olmoe.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    cur = None
    for line in open(path):
        line = line.rstrip("\n")
        if line.startswith("kernel: "):
            cur = line[len("kernel: "):].strip()
            fields[cur] = {}
        elif cur and ":" in line:
            key, val = line.split(":", 1)
            fields[cur][key.strip()] = val.strip()
    rec = fields.get(kernel)
    if not rec or rec.get("gemm_source_sha256") != sha:
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="olmoe")
    ap.add_argument("--cpu-tokens", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_gating_amd._lib as L
    from mixture_experts_layer_gating_amd.layer import MoELayer
    from moe_inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    code = L.dtype_code(tdt)
    b = 2 if wl.dtype == "bf16" else 4
    log(f"[bench] generating inputs for {wl.name}")
    inp = make_inputs(wl)

    def up(a):
        return torch.from_numpy(a).to(tdt).to(dev).contiguous()

    x, wr, w1, w2, dy = up(inp.x), up(inp.wr), up(inp.w1), up(inp.w2), up(inp.dy)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    forced = None if inp.forced_idx is None else torch.from_numpy(inp.forced_idx).to(dev)
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=tdt, device=dev)

    def step():
        layer.forward(x, wr, w1, w2, bias=bias, forced_idx=forced)
        layer.backward(dy)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = []  # (name, start_event, end_event)

    class Span:
        def __init__(self, name):
            self.name = name

        def __enter__(self):
            self.s = torch.cuda.Event(enable_timing=True)
            self.s.record()

        def __exit__(self, *exc):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            events.append((self.name, self.s, e))

    layer.timer = Span
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    layer.timer = None
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = wl.T / ((t1 - t0) / args.steps)

    per_call = {}
    for name, s, e in events:
        per_call.setdefault(name, []).append(s.elapsed_time(e))
    work = call_work(wl, b)
    kernels = {}
    for name, ts in per_call.items():
        avg = sum(ts) / len(ts)
        fl, by = work[name]
        rec = {"ms": round(avg, 4)}
        if fl:
            rec["tflops"] = round(fl / (avg * 1e-3) / 1e12, 1)
            rec["frac_mfma"] = round(fl / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if by:
            rec["gbs"] = round(by / (avg * 1e-3) / 1e9, 1)
            rec["frac_hbm"] = round(by / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        if name in GEMM_CALLS:
            rec["kernel"] = kernel_name(L, name, wl, code)
        kernels[name] = rec

    # Grouped-GEMM share of the bf16 peak, over the six expert GEMM launches.
    g_fl = sum(work[n][0] for n in EXPERT_GEMMS)
    g_ms = sum(kernels[n]["ms"] for n in EXPERT_GEMMS)
    gemm_frac = g_fl / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS

    # Dominant kernel: the GEMM kernel instance with the largest time per step.
    by_kernel = {}
    for n in GEMM_CALLS:
        kname = kernels[n]["kernel"]
        agg = by_kernel.setdefault(kname, {"ms": 0.0, "flops": 0, "launches": 0})
        agg["ms"] += kernels[n]["ms"]
        agg["flops"] += work[n][0]
        agg["launches"] += 1
    dom, agg = max(by_kernel.items(), key=lambda kv: kv[1]["ms"])
    flops_per_launch = agg["flops"] / agg["launches"]
    avg_launch_ms = agg["ms"] / agg["launches"]
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": read_traffic(dom), "kernel": dom, "launches_per_step": agg["launches"],
                "flops_per_launch": flops_per_launch, "avg_launch_ms": round(avg_launch_ms, 4)}

    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy probe: 3 x 1 GiB device copies done")

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded normal inputs and weights)",
        "config": {"workload": f"{wl.name}: MoE layer T={wl.T} d={wl.d} E={wl.E} top-{wl.k} "
                               f"SwiGLU d_ff={wl.F}, fwd+bwd",
                   "T": wl.T, "d_model": wl.d, "experts": wl.E, "top_k": wl.k, "d_ff": wl.F,
                   "regime": wl.regime, "parallelism": "single GPU"},
        "grouped_gemm_frac_of_bf16_peak": round(gemm_frac, 4),
        "grouped_gemm_tflops": round(g_fl / (g_ms * 1e-3) / 1e12, 1),
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_tokens, wl.T))
    else:
        out["cpu_baseline"] = None
    del np
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
