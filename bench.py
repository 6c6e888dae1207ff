#!/usr/bin/env python
"""Benchmark: one forward+backward step of the sparse MoE layer on one MI355X.

Headline workload (default ``large``): the large-expert layer, T = 16384
tokens, d = 4096, E = 128 experts, top-8 softmax gate, SwiGLU experts with
d_ff = 1536, bf16 storage with fp32 accumulation, seeded synthetic inputs
resident in HBM before timing -- the largest of the single-GPU workloads.
After it, every other workload (OLMoE-like natural / log-Zipf skewed /
forced-uniform routing, sparse small groups, tiny fp32) is measured the same
way and reported as a sub-record of the same line.

A step is one pass of the whole path: router GEMM, top-k routing, token
counting / index generation, permutation (fused into GEMM 1's loads),
grouped GEMM 1 + SwiGLU, grouped GEMM 2, weighted combine, and the backward
pass of all of them (dx, dW1, dW2, d_router).  Prints ONE JSON line on
stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--configs a,b,... | --configs none]
                  [--cpu-tokens N | --no-cpu-baseline] [--copy-probe]

``--copy-probe`` adds a plain 1 GiB device copy (torch ``copy_``) after the
timed region, whose counters calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE.
"""
from __future__ import annotations

import argparse
import gc
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
HEADLINE = "large"
SUB_CONFIGS = ("olmoe", "olmoe_skew", "olmoe_uniform", "sparse", "tiny")
# Tokens of the CPU-oracle sample per workload (full weights; a few seconds
# of float32 NumPy per pass on 16 host cores).
CPU_TOKENS = {"large": 2048, "olmoe": 2048, "olmoe_skew": 2048, "olmoe_uniform": 2048,
              "sparse": 512, "tiny": 256}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- work model
def call_work(wl, b, gather_dy=False):
    """Algorithmic FLOPs and HBM bytes of each library call of one step.

    Bytes count each input read once and each output written once (``b`` =
    bytes per activation / weight element; indices and gate values 4 B).  A
    gathered operand counts as its permuted copy would (T*k rows).  With
    ``gather_dy`` the combine's backward writes no dyp, GEMM 2's backward
    reads dy through the row map with the sorted gate weights, and the SwiGLU
    backward also writes the scaled activation."""
    T, d, E, k, F = wl.T, wl.d, wl.E, wl.k, wl.F
    Tk = T * k
    f = {}
    f["router_fwd"] = (2 * T * d * E, T * d * b + d * E * b + T * E * 4)
    f["route_topk"] = (0, T * E * 4 * 2 + Tk * 8)
    f["count_index"] = (0, Tk * 4 * 2 + Tk * 4 * 2 + (E + 1) * 8)
    f["permute"] = (0, T * d * b + Tk * d * b + Tk * 4)
    f["gemm1_fwd"] = (2 * Tk * d * 2 * F, Tk * d * b + E * d * 2 * F * b + Tk * 2 * F * b)
    f["act_fwd"] = (0, Tk * 2 * F * b + Tk * F * b)
    f["act_fwd_recompute"] = f["act_fwd"]  # the same kernel, in the backward pass
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
    if gather_dy:
        f["unpermute_bwd"] = (0, T * d * b + Tk * d * b + Tk * 12)
        f["gather_scale"] = (0, Tk * 12)
        f["gemm2_bwd_da"] = (f["gemm2_bwd_da"][0], f["gemm2_bwd_da"][1] + Tk * 8)
        f["gemm2_bwd_dw"] = (f["gemm2_bwd_dw"][0], f["gemm2_bwd_dw"][1] + Tk * 4)
        f["act_bwd"] = (0, f["act_bwd"][1] + Tk * F * b + Tk * 4)
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
MOVE_CALLS = ("unpermute", "unpermute_bwd", "act_bwd", "permute_bwd")  # HBM-bound

GATHER_CALLS = ("gemm1_swiglu_fwd", "gemm1_bwd_dw")  # read x through src / k when gathering


def kernel_name(L, call, wl, code, gather=False, gather_dy=False):
    """Name (as rocprofv3 prints it) of the kernel a GEMM call launches."""
    prod, M, K, N, E = GEMM_CALLS[call](wl)
    plan = L.moe_grouped_gemm_plan(prod, M, K, N, E, code)
    if not plan["mfma"]:
        return f"gemm_f32_kernel<{prod}, ...>"
    out = "float" if prod == 2 or call == "router_fwd" else "unsigned short"
    mode = 0 if prod == 3 else prod
    glu = "true" if prod == 3 else "false"
    gx = "true" if ((gather and call in GATHER_CALLS)
                    or (gather_dy and call == "gemm2_bwd_da")) else "false"
    gy = "true" if gather_dy and call == "gemm2_bwd_dw" else "false"
    return (f"gemm_mfma_kernel<{mode}, {plan['tile_m']}, {plan['tile_n']}, "
            f"{plan['waves_m']}, {plan['waves_n']}, {out}, {glu}, {gx}, {gy}>")


def default_gather_dy(L, wl, code):
    """Whether the layer reads dy through the row map in GEMM 2's backward
    (its default wherever the bf16 MFMA path applies)."""
    return bool(L.moe_grouped_gemm_plan(1, wl.T * wl.k, wl.F, wl.d, wl.E, code)["mfma"])


# ---------------------------------------------------------------- CPU baseline
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(inp, tokens, reps=3):
    """Time the CPU oracle (float32 NumPy, the oracle's own definitions in its
    float32 precision mode) on the first ``tokens`` tokens of the same
    workload with the full weights: forward + backward, ``reps`` passes; the
    median pass gives the rate."""
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
    times = []
    with threadpool_limits(limits=cores), O.precision(np.float32):
        info = threadpool_info()
        used = max([i.get("num_threads", 1) for i in info] or [1])
        x = inp.x[t]
        forced = None if inp.forced_idx is None else inp.forced_idx[t]
        for _ in range(reps):
            t0 = time.perf_counter()
            fwd = O.layer_forward(x, inp.wr, inp.w1, inp.w2, wl.k, bias=inp.bias,
                                  forced_idx=forced)
            O.layer_backward(fwd, inp.dy[t], x, inp.wr, inp.w1, inp.w2, wl.k)
            times.append(time.perf_counter() - t0)
            del fwd
    times.sort()
    med = times[len(times) // 2]
    flops = 18 * tokens * wl.k * wl.d * wl.F + 6 * tokens * wl.d * wl.E
    return {"value": round(tokens / med, 3), "unit": "tokens/s", "cores": int(used),
            "kind": "oracle", "cpu_model": cpu_model(),
            "gflops": round(flops / med / 1e9, 1),
            "sample": (f"{tokens} of {wl.T} tokens of the same layer (full weights), "
                       f"float32 NumPy oracle forward+backward, median of {reps} passes "
                       f"({', '.join('%.2f' % v for v in times)} s)")}


# ---------------------------------------------------------------- traffic
def traffic_file(workload):
    return os.path.join(PROFILES, f"gemm_traffic_{workload}.txt")


def read_traffic(kernel, workload):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 --pmc
    summary of ``workload``, if that summary was taken on the current
    grouped-GEMM source."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
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


# ---------------------------------------------------------------- profile summaries
def _csv_rows(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _short(name):
    name = name.replace("(anonymous namespace)::", "").replace("moe::", "")
    return name.split("(")[0].replace("void ", "").strip()


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


def _per_kernel(directory, counter):
    res = {}
    for r in _csv_rows(directory, "_counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        res.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return res


def summarize_pmc(fetch_dir, write_dir, out, command, command2, workload):
    """HBM traffic per launch of each grouped-GEMM kernel from two rocprofv3
    --pmc passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by
    the counter's reading on the 1 GiB device copies of --copy-probe."""
    from moe_inputs import WORKLOADS
    fetch = _per_kernel(fetch_dir, "FETCH_SIZE")
    write = _per_kernel(write_dir, "WRITE_SIZE")
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
    wl = WORKLOADS[workload]
    import mixture_experts_layer_gating_amd._lib as L
    code = L.MOE_BF16 if wl.dtype == "bf16" else L.MOE_F32
    work = call_work(wl, 2 if wl.dtype == "bf16" else 4, default_gather_dy(L, wl, code))
    lines = [f"# HBM traffic of the grouped-GEMM kernels (rocprofv3 --pmc), workload {workload}",
             "",
             f"command (FETCH_SIZE pass): {command}",
             f"command (WRITE_SIZE pass): {command2}",
             "",
             f"calibration: 1 GiB device copy reads FETCH_SIZE {sum(cf) / len(cf):.0f} KiB, "
             f"WRITE_SIZE {sum(cw) / len(cw):.0f} KiB per dispatch",
             f"scale factors: fetch x{f_fetch:.4f}, write x{f_write:.4f}", ""]
    names = _kernel_calls(wl)
    for name in sorted(fetch):
        if "gemm_mfma_kernel" not in name or name not in write:
            continue
        short = _short(name)
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write[name]) / len(write[name])
        traffic = fk * 1024 * f_fetch + wk * 1024 * f_write
        calls = names.get(short, [])
        alg = sum(work[c][1] for c in calls) / len(calls) if calls else 0
        lines += [f"kernel: {short}",
                  f"  calls: {', '.join(calls) if calls else '?'}",
                  f"  dispatches: {len(fetch[name])}",
                  f"  fetch_kib_per_dispatch: {fk:.1f}",
                  f"  write_kib_per_dispatch: {wk:.1f}",
                  f"  traffic_bytes_per_launch: {traffic:.0f}",
                  f"  algorithmic_bytes_per_launch: {alg:.0f}",
                  f"  traffic_over_algorithmic: {traffic / alg:.3f}" if alg else
                  "  traffic_over_algorithmic: ?",
                  f"  gemm_source_sha256: {sha}", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _kernel_calls(wl):
    """Kernel name -> the GEMM calls of one step that launch it (host-only
    plan queries; gathered GEMM 1 / dW1 as the layer runs them)."""
    import mixture_experts_layer_gating_amd._lib as L
    code = L.MOE_BF16 if wl.dtype == "bf16" else L.MOE_F32
    plan = L.moe_grouped_gemm_plan(3, wl.T * wl.k, wl.d, 2 * wl.F, wl.E, code)
    gather = bool(plan["mfma"])
    gdy = default_gather_dy(L, wl, code)
    calls = [c for c in GEMM_CALLS if c not in ("gemm1_fwd",)]
    out = {}
    for c in calls:
        out.setdefault(kernel_name(L, c, wl, code, gather, gdy), []).append(c)
    return out


def summarize_busy(directory, trace_dir, out, command, command_trace, workload):
    """Effective clock and MFMA activity per grouped-GEMM kernel from one
    --pmc pass (GRBM_GUI_ACTIVE, SQ_BUSY_CYCLES, SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_VALU_MFMA_MOPS_BF16) and the average kernel durations of a
    --kernel-trace --stats run of the same command."""
    from moe_inputs import WORKLOADS
    counters = ("GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
                "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    vals = {c: _per_kernel(directory, c) for c in counters}
    # Each dispatch's own duration in the (serialised) counter pass, for the
    # clock: GRBM_GUI_ACTIVE counts the cycles of that same interval.
    pmc_ns = {}
    for r in _csv_rows(directory, "_counter_collection.csv"):
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            pmc_ns.setdefault(r["Kernel_Name"], []).append(
                float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    durs = {}
    for r in _csv_rows(trace_dir, "_kernel_stats.csv"):
        durs[_short(r["Name"])] = float(r["AverageNs"])
    wl = WORKLOADS[workload]
    import mixture_experts_layer_gating_amd._lib as L
    work = call_work(wl, 2, default_gather_dy(L, wl, L.MOE_BF16))
    names = _kernel_calls(wl)
    lines = [f"# Clock and MFMA activity of the grouped-GEMM kernels, workload {workload}", "",
             f"command (--pmc pass): {command}",
             f"command (--kernel-trace --stats pass): {command_trace}", "",
             "Per dispatch (mean over dispatches).  GRBM_GUI_ACTIVE is summed over the 8 XCDs "
             "(the agent reports Num_Xcc 8, 1024 SIMDs, max engine clock 2400 MHz): busy "
             "cycles per XCD = GRBM_GUI_ACTIVE / 8, effective clock = that / the dispatch's "
             "own duration in the counter pass (its start and end timestamps; dispatches are "
             "serialised there).  SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs, so MFMA "
             "busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs) is the "
             "fraction of the chip's MFMA issue slots at the clock it ran at, and clock / "
             "2.4 GHz x MFMA busy is the fraction of the 2.5 PFLOP/s peak.  'trace avg us' is "
             "the kernel's average duration in the --kernel-trace --stats pass (kernels of "
             "one call per row only when the kernel serves one call).  executed / "
             "algorithmic = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / algorithmic FLOPs.", "",
             "| kernel (calls) | dispatches | trace avg us | counter-pass us | "
             "GRBM_GUI_ACTIVE / 8 | clock GHz | SQ_BUSY_CYCLES | MFMA busy cycles | MFMA busy | "
             "clock/2.4 x busy | executed / algorithmic |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name in sorted(vals["GRBM_GUI_ACTIVE"]):
        lib = name.startswith("Cijk")  # the library GEMM of the reference product
        if "gemm_mfma_kernel" not in name and not lib:
            continue
        short = "hipBLASLt bf16 8192^3 (torch.matmul)" if lib else _short(name)
        mean = {c: (sum(vals[c].get(name, [0])) / max(1, len(vals[c].get(name, [0]))))
                for c in counters}
        dur = durs.get(_short(name))
        calls = names.get(short, [])
        alg = sum(work[c][0] for c in calls) / len(calls) if calls else 0
        if lib:
            calls, alg = ["library reference"], 2.0 * 8192 ** 3
        act = mean["GRBM_GUI_ACTIVE"] / 8
        pns = pmc_ns.get(name, [])
        pdur = sum(pns) / len(pns) if pns else 0.0
        clock = act / pdur if pdur else float("nan")
        busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (act * 1024) if act else float("nan")
        ratio = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / alg if alg else float("nan")
        lines.append(f"| {short} ({', '.join(calls)}) | {len(vals['GRBM_GUI_ACTIVE'][name])} | "
                     f"{(dur or 0) / 1e3:.1f} | {pdur / 1e3:.1f} | {act:.0f} | {clock:.3f} | "
                     f"{mean['SQ_BUSY_CYCLES']:.0f} | {mean['SQ_VALU_MFMA_BUSY_CYCLES']:.0f} | "
                     f"{busy:.3f} | {clock / 2.4 * busy:.3f} | {ratio:.3f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


# ---------------------------------------------------------------- GPU timing
class Recorder:
    """Event spans around the layer's calls (all of them, or only `names`),
    recorded on the stream each call is launched on."""

    def __init__(self, torch, names=None):
        self.torch = torch
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


def roofline_of(work, calls, avg_launch_ms):
    """Roofline record of a kernel serving ``calls`` (per launch: algorithmic
    work averaged over the calls, over the average launch time).  The bound
    is the roof under which its algorithmic intensity falls: MFMA above the
    ridge point (peak FLOP/s over peak bytes/s, ~312 FLOP/B), HBM below it."""
    flops = sum(work[n][0] for n in calls) / len(calls)
    nbytes = sum(work[n][1] for n in calls) / len(calls)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / nbytes >= ridge:
        achieved = flops / (avg_launch_ms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = nbytes / (avg_launch_ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
             "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    r.update({"flops_per_launch": flops, "bytes_per_launch": nbytes})
    return r


def measure(wl, args, detail):
    """Time one workload: K back-to-back steps (the rate), the dominant
    kernel's launches inside them (HIP events on the launch stream), per-step
    medians warm and after an L2/MALL flush, and a per-call breakdown pass.
    ``detail`` adds the two-stream variant and the library-GEMM reference."""
    import numpy as np  # noqa: F401
    import torch

    import mixture_experts_layer_gating_amd._lib as L
    from mixture_experts_layer_gating_amd.layer import MoELayer
    from moe_inputs import make_inputs

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    code = L.dtype_code(tdt)
    b = 2 if wl.dtype == "bf16" else 4
    log(f"[bench] {wl.name}: generating inputs")
    inp = make_inputs(wl)

    def up(a):
        return torch.from_numpy(a).to(tdt).to(dev).contiguous()

    x, wr, w1, w2, dy = up(inp.x), up(inp.wr), up(inp.w1), up(inp.w2), up(inp.dy)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    forced = None if inp.forced_idx is None else torch.from_numpy(inp.forced_idx).to(dev)
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=tdt, device=dev,
                     overlap_wgrad=args.overlap_wgrad and detail,
                     gather_dy=not args.no_gather_dy)
    work = call_work(wl, b, layer.gather_dy)

    def step():
        layer.forward(x, wr, w1, w2, bias=bias, forced_idx=forced)
        layer.backward(dy)

    # Warm-up, with every call timed: the per-call times pick the dominant
    # kernel, the only one whose calls carry events in the timed region (an
    # event pair costs the stream a few microseconds; ~40 of them per step
    # would inflate a short step by ~4%).
    log(f"[bench] {wl.name}: warmup {args.warmup}")
    warm = Recorder(torch)
    layer.timer = warm.span
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    layer.timer = None
    warm_ms = warm.per_call_ms()
    kname = {n: kernel_name(L, n, wl, code, layer.gather_x, layer.gather_dy)
             for n in GEMM_CALLS if n in warm_ms}
    by_kernel = {}
    for n, kn in kname.items():
        by_kernel.setdefault(kn, []).append(n)
    dom = max(by_kernel, key=lambda kn: sum(warm_ms[n] for n in by_kernel[kn]))
    dom_calls = by_kernel[dom]

    log(f"[bench] {wl.name}: timing {args.steps} steps (events on {', '.join(dom_calls)})")
    timed = Recorder(torch, set(dom_calls))
    graph = None
    if args.graph and detail:
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
    dom_ms = timed.per_call_ms() if graph is None else None
    if dom_ms is None:  # graph mode: one eager step with events on the dominant calls
        probe = Recorder(torch, set(dom_calls))
        layer.timer = probe.span
        step()
        torch.cuda.synchronize()
        layer.timer = None
        dom_ms = probe.per_call_ms()
    avg_launch_ms = sum(dom_ms[n] for n in dom_calls) / len(dom_calls)
    roofline = roofline_of(work, dom_calls, avg_launch_ms)
    roofline.update({"traffic": read_traffic(dom, wl.name), "kernel": dom,
                     "calls": dom_calls, "launches_per_step": len(dom_calls),
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
    step_median["tokens_per_s_after_cache_flush"] = round(
        wl.T / (step_median["after_cache_flush_ms"] * 1e-3), 1)

    # Per-call breakdown: a separate pass after the timed region, every call timed.
    n_brk = min(args.steps, 10)
    log(f"[bench] {wl.name}: per-call breakdown over {n_brk} further steps")
    brk = Recorder(torch)
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
            rec["kernel"] = kernel_name(L, name, wl, code, layer.gather_x, layer.gather_dy)
        kernels[name] = rec

    # Grouped-GEMM share of the bf16 peak, over the six expert GEMM launches.
    g_fl = sum(work[n][0] for n in EXPERT_GEMMS)
    g_ms = sum(kernels[n]["ms"] for n in EXPERT_GEMMS)
    rec = {
        "workload": (f"{wl.name}: MoE layer T={wl.T} d={wl.d} E={wl.E} top-{wl.k} "
                     f"SwiGLU d_ff={wl.F} {wl.dtype}, {wl.regime} routing, fwd+bwd"),
        "ms_per_step": round(ms_per_step, 4),
        "tokens_per_s": round(wl.T / (ms_per_step * 1e-3), 1),
        "step_tflops": round((g_fl + sum(work[n][0] for n in ("router_fwd", "router_bwd_da",
                                                              "router_bwd_dw")))
                             / (ms_per_step * 1e-3) / 1e12, 1),
        "grouped_gemm_frac_of_bf16_peak": round(g_fl / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                                4),
        "grouped_gemm_tflops": round(g_fl / (g_ms * 1e-3) / 1e12, 1),
        "data_movement_frac_of_hbm": {n: kernels[n]["frac_hbm"] for n in MOVE_CALLS
                                      if n in kernels},
        "roofline": roofline,
        "step_median": step_median,
        "kernels": kernels,
    }
    if wl.dtype != "bf16":
        rec["note"] = ("float32 layer: float32-MFMA kernels (no bf16 path); the bf16 "
                       "fractions do not apply")

    if detail and not args.overlap_wgrad and not args.graph and not args.no_overlap_variant:
        # The same step with the expert weight-gradient GEMMs on a second
        # stream (beside the data-gradient chain), timed after everything
        # above so that the per-kernel figures stay those of one stream.
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
        rec["overlap_wgrad"] = {
            "ms_per_step": round(o_ms, 4), "tokens_per_s": round(wl.T / (o_ms * 1e-3), 1),
            "note": "weight-gradient GEMMs on a second stream; not the headline: "
                    "overlapped kernels stretch each other's measured durations"}
        del lay2

    if (detail or wl.name == "olmoe") and not args.no_overlap_variant:
        # Selective recomputation (activation checkpointing of the layer):
        # what each mode keeps between the passes, and its step time.
        lay3 = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=tdt, device=dev)
        rc = {}
        for mode in MoELayer.RECOMPUTE:
            lay3.recompute = mode

            def step3():
                lay3.forward(x, wr, w1, w2, bias=bias, forced_idx=forced)
                lay3.backward(dy)

            for _ in range(max(1, args.warmup)):
                step3()
            torch.cuda.synchronize()
            r0 = time.perf_counter()
            for _ in range(args.steps):
                step3()
            torch.cuda.synchronize()
            r_ms = (time.perf_counter() - r0) * 1e3 / args.steps
            rc[mode] = {"ms_per_step": round(r_ms, 4),
                        "saved_bytes": int(sum(lay3.saved_bytes(mode).values()))}
        for mode in ("act", "layer"):
            rc[mode]["time_cost_pct"] = round(
                100 * (rc[mode]["ms_per_step"] / rc["none"]["ms_per_step"] - 1), 2)
            rc[mode]["memory_saved_bytes"] = rc["none"]["saved_bytes"] - rc[mode]["saved_bytes"]
        rec["recompute"] = rc
        del lay3

    if detail and args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy probe: 3 x 1 GiB device copies done")
        del src, dst

    del layer, x, wr, w1, w2, dy, bias, forced, graph
    gc.collect()
    torch.cuda.empty_cache()
    return rec, inp


def library_gemm_reference(torch, own=True):
    """What a plain library GEMM (torch.matmul, hipBLASLt) sustains on this
    box for a large square bf16 product: context for the MFMA roofline.  With
    ``own``, this library's grouped GEMM runs the same product as a single
    group (the forward NN kernel, and the NT kernel of the data gradient), so
    the two kernels are compared on a shape with no expert structure."""
    dev = torch.device("cuda:0")
    n = 8192
    ga = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    gb = torch.randn(n, n, device=dev, dtype=torch.bfloat16)

    def tflops(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 2 * n ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12

    lib = tflops(lambda: torch.matmul(ga, gb))
    res = {"what": "torch.matmul (hipBLASLt) bf16 8192 x 8192 x 8192",
           "tflops": round(lib, 1), "frac_of_peak": round(lib / PEAK_BF16_TFLOPS, 4)}
    if own:
        import mixture_experts_layer_gating_amd._lib as L
        off = torch.tensor([0, n], dtype=torch.int32, device=dev)
        gc_ = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        b3 = gb.view(1, n, n)
        nn = tflops(lambda: L.moe_grouped_gemm_fwd(ga, b3, off, n, n, n, 1, L.MOE_BF16, gc_,
                                                   L.MOE_BF16))
        nt = tflops(lambda: L.moe_grouped_gemm_bwd(None, b3, ga, off, n, n, n, 1, L.MOE_BF16,
                                                   gc_, None, None, None, 0))
        res["this_library_one_group"] = {
            "what": "moe_grouped_gemm_fwd (NN) and moe_grouped_gemm_bwd data gradient (NT), "
                    "one group, bf16 8192 x 8192 x 8192",
            "nn_tflops": round(nn, 1), "nt_tflops": round(nt, 1),
            "nn_frac_of_peak": round(nn / PEAK_BF16_TFLOPS, 4),
            "nt_frac_of_peak": round(nt / PEAK_BF16_TFLOPS, 4)}
        del gc_
    del ga, gb
    return res


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--configs", default=",".join(SUB_CONFIGS),
                    help="comma-separated workloads measured after the headline one "
                         "('none' for none)")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the headline CPU-oracle sample (default per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--overlap-wgrad", action="store_true",
                    help="expert weight-gradient GEMMs on a second stream (headline workload)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured as a HIP graph (headline "
                         "workload; per-kernel figures still come from eager steps)")
    ap.add_argument("--no-overlap-variant", action="store_true",
                    help="skip the two-stream variant of the headline workload (profiling "
                         "runs: overlapped kernels stretch each other's durations)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--no-gather-dy", action="store_true",
                    help="write the combine's gradient dyp and run GEMM 2's backward on it "
                         "(MoELayer(gather_dy=False)) instead of reading dy through the row map")
    ap.add_argument("--no-own-dense", action="store_true",
                    help="leave this library's one-group GEMMs out of the library reference "
                         "(profiling passes: they would add dispatches to the expert kernels)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write a text summary of a rocprofv3 --kernel-trace --stats output")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write HBM traffic per grouped-GEMM launch from two --pmc outputs")
    ap.add_argument("--summarize-busy", nargs=2, metavar=("PMC_DIR", "TRACE_DIR"),
                    help="write clock and MFMA activity per grouped-GEMM kernel")
    ap.add_argument("--out", help="summary file to write")
    ap.add_argument("--command", default="", help="profiled command, recorded in the summary")
    ap.add_argument("--command2", default="", help="second profiled command")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.out, args.command,
                      args.command2, args.workload)
        return
    if args.summarize_busy:
        summarize_busy(args.summarize_busy[0], args.summarize_busy[1], args.out, args.command,
                       args.command2, args.workload)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_layer_gating_amd._lib  # noqa: F401  (raises if not built)
    from moe_inputs import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = WORKLOADS[args.workload]
    subs = [] if args.configs in ("", "none") else [c for c in args.configs.split(",")
                                                    if c != wl.name]
    for c in subs:
        if c not in WORKLOADS:
            raise SystemExit(f"unknown workload {c}")

    def cpu_leg(inp, tokens):
        if args.no_cpu_baseline:
            return None
        tokens = min(tokens, inp.wl.T)
        log(f"[bench] cpu baseline ({inp.wl.name}): float32 oracle on {tokens} tokens")
        return cpu_baseline(inp, tokens)

    head, inp = measure(wl, args, detail=True)
    ref_gemm = (library_gemm_reference(torch, own=not args.no_own_dense)
                if wl.dtype == "bf16" else None)
    head_cpu = cpu_leg(inp, args.cpu_tokens or CPU_TOKENS.get(wl.name, 1024))
    del inp
    configs = {}
    for c in subs:
        configs[c], inp = measure(WORKLOADS[c], args, detail=False)
        configs[c]["cpu_baseline"] = cpu_leg(inp, CPU_TOKENS.get(c, 1024))
        del inp
        gc.collect()

    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded normal inputs and weights)",
        "config": {"workload": head["workload"],
                   "T": wl.T, "d_model": wl.d, "experts": wl.E, "top_k": wl.k, "d_ff": wl.F,
                   "regime": wl.regime, "parallelism": "single GPU",
                   "streams": 2 if args.overlap_wgrad else 1,
                   "launch": "hip graph replay" if args.graph else "eager"},
        "value_note": ("value = tokens/s over the K timed steps run back to back (inputs "
                       "resident in HBM); step_median.tokens_per_s_after_cache_flush is the "
                       "rate with L2 and MALL flushed before every step"),
        "grouped_gemm_frac_of_bf16_peak": head["grouped_gemm_frac_of_bf16_peak"],
        "grouped_gemm_tflops": head["grouped_gemm_tflops"],
        "step_tflops": head["step_tflops"],
        "roofline": head["roofline"],
        "step_median": head["step_median"],
        "data_movement_frac_of_hbm": head["data_movement_frac_of_hbm"],
        "overlap_wgrad": head.get("overlap_wgrad"),
        "recompute": head.get("recompute"),
        "library_gemm_reference": ref_gemm,
        "kernels": head["kernels"],
        "kernels_note": "per-call times from a pass of steps after the timed region",
        "configs": configs,
    }
    out["cpu_baseline"] = head_cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
