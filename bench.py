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
    f["gemm1_swiglu_fwd"] = (f["gemm1_fwd"][0], f["gemm1_fwd"][1] + Tk * F * b)
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
    "gemm1_swiglu_fwd": lambda wl: (3, wl.T * wl.k, wl.d, 2 * wl.F, wl.E),
    "gemm2_fwd": lambda wl: (0, wl.T * wl.k, wl.F, wl.d, wl.E),
    "gemm2_bwd_da": lambda wl: (1, wl.T * wl.k, wl.F, wl.d, wl.E),
    "gemm2_bwd_dw": lambda wl: (2, wl.T * wl.k, wl.F, wl.d, wl.E),
    "gemm1_bwd_da": lambda wl: (1, wl.T * wl.k, wl.d, 2 * wl.F, wl.E),
    "gemm1_bwd_dw": lambda wl: (2, wl.T * wl.k, wl.d, 2 * wl.F, wl.E),
    "router_bwd_da": lambda wl: (1, wl.T, wl.d, wl.E, 1),
    "router_bwd_dw": lambda wl: (2, wl.T, wl.d, wl.E, 1),
}
EXPERT_GEMMS = ("gemm1_swiglu_fwd", "gemm2_fwd", "gemm2_bwd_da", "gemm2_bwd_dw",
                "gemm1_bwd_da", "gemm1_bwd_dw")


GATHER_CALLS = ("gemm1_swiglu_fwd", "gemm1_bwd_dw")  # read x through src / k when gathering


def kernel_name(L, call, wl, code, gather=False):
    """Name (as rocprofv3 prints it) of the kernel a GEMM call launches."""
    prod, M, K, N, E = GEMM_CALLS[call](wl)
    plan = L.moe_grouped_gemm_plan(prod, M, K, N, E, code)
    if not plan["mfma"]:
        return f"gemm_simt_kernel<{prod}, ...>"
    out = "float" if prod == 2 or call == "router_fwd" else "unsigned short"
    mode = 0 if prod == 3 else prod
    glu = "true" if prod == 3 else "false"
    gx = "true" if gather and call in GATHER_CALLS else "false"
    return (f"gemm_mfma_kernel<{mode}, {plan['tile_m']}, {plan['tile_n']}, "
            f"{plan['waves_m']}, {plan['waves_n']}, {out}, {glu}, {gx}>")


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(inp, tokens, reps=2):
    """Time the CPU oracle (float64 NumPy, as it stands) on the first
    ``tokens`` tokens of the same workload: forward + backward, ``reps``
    times; reports the mean rate."""
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
        forced = None if inp.forced_idx is None else inp.forced_idx[t]
        t0 = time.perf_counter()
        for _ in range(reps):
            fwd = O.layer_forward(x, inp.wr, inp.w1, inp.w2, wl.k, bias=inp.bias,
                                  forced_idx=forced)
            O.layer_backward(fwd, inp.dy[t], x, inp.wr, inp.w1, inp.w2, wl.k)
            del fwd
        dt = time.perf_counter() - t0
    return {"value": round(tokens * reps / dt, 3), "unit": "tokens/s", "cores": int(used),
            "kind": "oracle",
            "sample": (f"{tokens} of {wl.T} tokens of the same layer (full weights), "
                       f"float64 NumPy forward+backward, {reps} passes, {dt:.1f} s")}


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
    rec = None
    for name, r in fields.items():
        if name.startswith(kernel.split("<")[0]) and kernel.split("<")[1] in name:
            rec = r
    if not rec or rec.get("gemm_source_sha256") != sha:
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- profile summaries
def _csv_rows(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def summarize_trace(directory, out, command):
    """Text summary of a rocprofv3 --kernel-trace --stats run."""
    rows = _csv_rows(directory, "_kernel_stats.csv")
    lines = ["# rocprofv3 kernel statistics", "", f"command: {command}", "",
             "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").replace("moe::", "")
        name = name.split("(moe::")[0].split("(char")[0].split("(float")[0].split("(int")[0]
        name = name.split("(unsigned")[0].strip()
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_pmc(fetch_dir, write_dir, out, command, command2):
    """HBM traffic per launch of each grouped-GEMM kernel from two rocprofv3
    --pmc passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by
    the counter's reading on the 1 GiB device copies of --copy-probe."""
    def per_kernel(directory, counter):
        res = {}
        for r in _csv_rows(directory, "_counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            res.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return res
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    # the 1 GiB copies are the copyBuffer dispatches that write ~1 GiB
    copies = [i for i, v in enumerate(write.get("__amd_rocclr_copyBuffer", []))
              if abs(v - gib_kib) < 0.25 * gib_kib]
    if not copies:
        raise SystemExit("no 1 GiB copy dispatches found (run bench.py with --copy-probe)")
    cf = [fetch["__amd_rocclr_copyBuffer"][i] for i in copies]
    cw = [write["__amd_rocclr_copyBuffer"][i] for i in copies]
    f_fetch = gib_kib / (sum(cf) / len(cf))
    f_write = gib_kib / (sum(cw) / len(cw))
    sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    lines = ["# HBM traffic of the grouped-GEMM kernels (rocprofv3 --pmc)", "",
             f"command (FETCH_SIZE pass): {command}",
             f"command (WRITE_SIZE pass): {command2}",
             "",
             f"calibration: 1 GiB device copy reads FETCH_SIZE {sum(cf) / len(cf):.0f} KiB, "
             f"WRITE_SIZE {sum(cw) / len(cw):.0f} KiB per dispatch",
             f"scale factors: fetch x{f_fetch:.4f}, write x{f_write:.4f}", ""]
    for name in sorted(fetch):
        if "gemm_mfma_kernel" not in name or name not in write:
            continue
        short = name.replace("(anonymous namespace)::", "").replace("moe::", "")
        short = short.split("(")[0].replace("void ", "").strip()
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write[name]) / len(write[name])
        traffic = fk * 1024 * f_fetch + wk * 1024 * f_write
        lines += [f"kernel: {short}",
                  f"  dispatches: {len(fetch[name])}",
                  f"  fetch_kib_per_dispatch: {fk:.1f}",
                  f"  write_kib_per_dispatch: {wk:.1f}",
                  f"  traffic_bytes_per_launch: {traffic:.0f}",
                  f"  gemm_source_sha256: {sha}", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="olmoe")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the CPU-oracle sample (default: the whole workload; "
                         "two passes take about 15 s on 16 host cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--overlap-wgrad", action="store_true",
                    help="expert weight-gradient GEMMs on a second stream")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured as a HIP graph (per-kernel "
                         "figures still come from eager steps)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write a text summary of a rocprofv3 --kernel-trace --stats output")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write HBM traffic per grouped-GEMM launch from two --pmc outputs")
    ap.add_argument("--out", help="summary file to write")
    ap.add_argument("--command", default="", help="profiled command, recorded in the summary")
    ap.add_argument("--command2", default="", help="second profiled command (WRITE_SIZE pass)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.out, args.command,
                      args.command2)
        return

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
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=tdt, device=dev,
                     overlap_wgrad=args.overlap_wgrad)
    work = call_work(wl, b)

    def step():
        layer.forward(x, wr, w1, w2, bias=bias, forced_idx=forced)
        layer.backward(dy)

    class Recorder:
        """Event spans around the layer's calls (all of them, or only `names`)."""

        def __init__(self, names=None):
            self.names = names
            self.events = []  # (name, start_event, end_event)
            rec = self

            class Span:
                def __init__(self, name):
                    self.name = name
                    self.on = rec.names is None or name in rec.names

                def __enter__(self):
                    if self.on:
                        self.s = torch.cuda.Event(enable_timing=True)
                        self.s.record()

                def __exit__(self, *exc):
                    if self.on:
                        e = torch.cuda.Event(enable_timing=True)
                        e.record()
                        rec.events.append((self.name, self.s, e))

            self.span = Span

        def per_call_ms(self):
            per = {}
            for name, s0, e in self.events:
                per.setdefault(name, []).append(s0.elapsed_time(e))
            return {n: sum(v) / len(v) for n, v in per.items()}

    # Warm-up, with every call timed: the per-call times pick the dominant
    # kernel, the only one whose calls carry events in the timed region (an
    # event pair costs the stream a few microseconds; ~40 of them per step
    # would inflate the step time by ~4%).
    log(f"[bench] warmup {args.warmup}")
    warm = Recorder()
    layer.timer = warm.span
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    layer.timer = None
    if not warm.events:  # --warmup 0: one untimed step to find the dominant kernel
        layer.timer = warm.span
        step()
        torch.cuda.synchronize()
        layer.timer = None
    warm_ms = warm.per_call_ms()
    kname = {n: kernel_name(L, n, wl, code, layer.gather_x) for n in GEMM_CALLS if n in warm_ms}
    by_kernel = {}
    for n, kn in kname.items():
        by_kernel.setdefault(kn, []).append(n)
    dom = max(by_kernel, key=lambda kn: sum(warm_ms[n] for n in by_kernel[kn]))
    dom_calls = by_kernel[dom]

    log(f"[bench] timing {args.steps} steps (events on {', '.join(dom_calls)})")
    timed = Recorder(set(dom_calls))
    graph = None
    if args.graph:
        # The whole step as one HIP graph over the same input buffers (no
        # events inside it: the dominant kernel is then timed in the
        # breakdown pass below).
        graph = layer.capture(x, wr, w1, w2, dy, bias=bias, forced_idx=forced)
        for _ in range(max(1, args.warmup)):
            graph.replay()
    else:
        layer.timer = timed.span
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    layer.timer = None
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = wl.T / ((t1 - t0) / args.steps)

    # Dominant kernel, from the events of the timed region.  Its bound is the
    # roof its algorithmic intensity falls under: MFMA above the ridge point
    # (peak FLOP/s over peak bytes/s, ~312 FLOP/B), HBM below it (tiny
    # groups, where the GEMMs stream weights and weight gradients).
    dom_ms = timed.per_call_ms() if graph is None else None
    flops_per_launch = sum(work[n][0] for n in dom_calls) / len(dom_calls)
    bytes_per_launch = sum(work[n][1] for n in dom_calls) / len(dom_calls)
    if dom_ms is None:  # graph mode: one eager step with events on the dominant calls
        probe = Recorder(set(dom_calls))
        layer.timer = probe.span
        step()
        torch.cuda.synchronize()
        layer.timer = None
        dom_ms = probe.per_call_ms()
    avg_launch_ms = sum(dom_ms[n] for n in dom_calls) / len(dom_calls)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops_per_launch / bytes_per_launch >= ridge:
        achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roofline.update({"traffic": read_traffic(dom) if wl.name == "olmoe" else None,
                     "kernel": dom, "launches_per_step": len(dom_calls),
                     "flops_per_launch": flops_per_launch, "bytes_per_launch": bytes_per_launch,
                     "avg_launch_ms": round(avg_launch_ms, 4)})

    # Per-step medians (HIP events around each step): steps back to back,
    # and steps each preceded by a 1 GiB write that flushes L2 and the MALL.
    def step_medians(n, flush):
        buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if flush else None
        times = []
        for _ in range(n):
            if buf is not None:
                buf.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if graph is not None:
                graph.replay()
            else:
                step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del buf
        times.sort()
        return round(times[len(times) // 2], 4)

    n_med = min(args.steps, 10)
    step_median = {"warm_ms": step_medians(n_med, False),
                   "after_cache_flush_ms": step_medians(n_med, True), "steps": n_med}

    # Per-call breakdown: a separate pass after the timed region, every call timed.
    n_brk = min(args.steps, 10)
    log(f"[bench] per-call breakdown over {n_brk} further steps")
    brk = Recorder()
    layer.timer = brk.span
    for _ in range(n_brk):
        step()
    torch.cuda.synchronize()
    layer.timer = None
    kernels = {}
    for name, avg in brk.per_call_ms().items():
        fl, by = work[name]
        rec = {"ms": round(avg, 4)}
        if fl:
            rec["tflops"] = round(fl / (avg * 1e-3) / 1e12, 1)
            rec["frac_mfma"] = round(fl / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if by:
            rec["gbs"] = round(by / (avg * 1e-3) / 1e9, 1)
            rec["frac_hbm"] = round(by / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        if name in GEMM_CALLS:
            rec["kernel"] = kernel_name(L, name, wl, code, layer.gather_x)
        kernels[name] = rec

    # Grouped-GEMM share of the bf16 peak, over the six expert GEMM launches.
    g_fl = sum(work[n][0] for n in EXPERT_GEMMS)
    g_ms = sum(kernels[n]["ms"] for n in EXPERT_GEMMS)
    gemm_frac = g_fl / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS

    # The same step with the expert weight-gradient GEMMs on a second stream
    # (beside the data-gradient chain), timed after everything above so that
    # the per-kernel figures stay those of the single-stream order.
    overlap = None
    if not args.overlap_wgrad and not args.graph:
        lay2 = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=tdt, device=dev, overlap_wgrad=True)

        def step2():
            lay2.forward(x, wr, w1, w2, bias=bias, forced_idx=forced)
            lay2.backward(dy)

        for _ in range(max(1, args.warmup)):
            step2()
        torch.cuda.synchronize()
        o0 = time.perf_counter()
        for _ in range(args.steps):
            step2()
        torch.cuda.synchronize()
        o_ms = (time.perf_counter() - o0) * 1e3 / args.steps
        overlap = {"ms_per_step": round(o_ms, 4), "tokens_per_s": round(wl.T / (o_ms * 1e-3), 1),
                   "note": "weight-gradient GEMMs on a second stream; not the headline: "
                           "overlapped kernels stretch each other's measured durations"}
        del lay2

    # Context for the MFMA roofline: what a plain library GEMM (torch.matmul,
    # hipBLASLt) sustains on this machine for a large square bf16 product.
    ref_gemm = None
    if wl.dtype == "bf16":
        n = 8192
        ga = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        gb = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(ga, gb)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.matmul(ga, gb)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        ref_gemm = {"what": "torch.matmul (hipBLASLt) bf16 8192 x 8192 x 8192",
                    "tflops": round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1),
                    "frac_of_peak": round(2 * n ** 3 / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del ga, gb

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
                   "regime": wl.regime, "parallelism": "single GPU",
                   "streams": 2 if args.overlap_wgrad else 1,
                   "launch": "hip graph replay" if args.graph else "eager"},
        "grouped_gemm_frac_of_bf16_peak": round(gemm_frac, 4),
        "grouped_gemm_tflops": round(g_fl / (g_ms * 1e-3) / 1e12, 1),
        "roofline": roofline,
        "step_median": step_median,
        "overlap_wgrad": overlap,
        "library_gemm_reference": ref_gemm,
        "kernels": kernels,
        "kernels_note": f"per-call times from {n_brk} steps after the timed region",
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: float64 oracle")
        out["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_tokens or wl.T, wl.T))
    else:
        out["cpu_baseline"] = None
    del np
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
