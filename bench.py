#!/usr/bin/env python3
"""MoE-layer forward benchmark on one MI355X.

A step is one forward pass of the whole layer -- router, top-k, gates, dispatch,
linear1 + SwiGLU, linear2 and the gate-weighted combine -- over one batch of seeded
synthetic tokens with random-init weights of the workload's shape, all resident in HBM
before timing starts.

With no workload named, the reported line is the DeepSeek-V3-shaped FP8 e4m3 x MXFP4
layer at T = 32768 tokens (the largest per-rank batch on the pages), and a `sweep` key in
the same line carries every other workload: the tiny fp32 layer (T = 64), the
Mixtral-shaped bf16 layer (T = 4096), the DeepSeek-V3-shaped bf16 layer (T = 8192), the
FP8 x MXFP4 layer at T = 512 and 8192 (and at 8192 with the sigmoid + Zipf-bias router,
dropless and with a capacity factor of 1.25), decode at T = 1 and 64 (whose metric is HBM
GB/s), the FP8 e4m3 x e4m3 layer at T = 8192, one expert-parallel rank's experts over the
rows 8 ranks send it, and the dense FP8 x MXFP4 GEMM.  Every entry carries its own
median / p10 / p90 step time, roofline of the dominant kernel, load statistics and
CPU-oracle rate (all host cores and one thread).

Both entry points compute the same layer: the persistent single-launch kernel
(moe_layer_fused) and the chain of step kernels (route, dispatch, ffn, combine).  Both
are timed; the faster gives an entry's value and each path's time is reported.

roofline: the dominant kernel's algorithmic work over its mean duration, measured with
HIP events on its own launch stream during a separate pass; `traffic` is that kernel's
HBM bytes per launch from hardware counters (profiles/traffic.txt), reported only while
the sources of that kernel still hash to the ones the counters were taken with.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# dense TFLOP/s (MI355X spec); FP8 x MXFP4 issues at the FP8 rate on this MFMA (measured), so
# both FP8 modes take the FP8 peak
PEAK = {"bf16": 2500.0, "fp8_mxfp4": 5000.0, "fp8_fp8": 5000.0, "f32": 157.3}
PEAK_HBM = 8000.0  # GB/s
METRIC = "MoE-layer active TFLOPS & tokens/s at T=1..32768 (bf16, FP8×FP4); GB/s at T=1"
DTYPE = {"f32": "f32", "bf16": "bf16", "fp8_mxfp4": "fp8e4m3 x mxfp4", "fp8_fp8": "fp8e4m3 x fp8e4m3"}
FP8 = ("fp8_mxfp4", "fp8_fp8")

# Entries of the default run, in execution order (entries that share weights run together).
# kind "layer": the whole layer on a workload at T tokens; "capacity": the same with the
# capacity-factor dispatch; "ep": one expert-parallel rank's experts over its receive
# buffer; "gemm": the dense FP8 x MXFP4 GEMM.  cpu / cpu1: CPU-oracle seconds on all host
# cores and on one thread.  The first entry is the headline.
HEADLINE = ("layer", "dsv3_fp8fp4", 32768)
SWEEP = [
    {"kind": "layer", "workload": "dsv3_fp8fp4", "T": 32768, "cpu": 12.0, "cpu1": 4.0},
    {"kind": "layer", "workload": "dsv3_fp8fp4", "T": 8192, "cpu": 4.0, "cpu1": 2.0},
    {"kind": "layer", "workload": "dsv3_fp8fp4", "T": 512, "cpu": 4.0, "cpu1": 2.0},
    {"kind": "layer", "workload": "dsv3_fp8fp4_zipf", "T": 8192, "cpu": 4.0, "cpu1": 2.0},
    {"kind": "capacity", "workload": "dsv3_fp8fp4_zipf", "T": 8192, "factor": 1.25, "cpu": 4.0, "cpu1": 2.0},
    {"kind": "layer", "workload": "decode_fp8fp4", "T": 1, "cpu": 2.0, "cpu1": 1.0},
    {"kind": "layer", "workload": "decode_fp8fp4", "T": 64, "cpu": 4.0, "cpu1": 2.0},
    {"kind": "ep", "workload": "dsv3_fp8fp4", "T": 8192, "E_local": 32, "n_src": 8, "cpu": 4.0, "cpu1": 2.0},
    {"kind": "gemm", "workload": "dsv3_fp8fp4", "M": 32768, "N": 4096, "K": 7168, "cpu": 3.0, "cpu1": 1.5},
    {"kind": "layer", "workload": "dsv3_fp8fp8", "T": 8192, "cpu": 4.0, "cpu1": 2.0},
    {"kind": "layer", "workload": "dsv3_bf16", "T": 8192, "cpu": 4.0, "cpu1": 2.0},
    {"kind": "layer", "workload": "mixtral_bf16", "T": 4096, "cpu": 4.0, "cpu1": 2.0},
    {"kind": "layer", "workload": "tiny_f32", "T": 64, "cpu": 2.0, "cpu1": 1.0},
]


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="measure one workload only: tiny_f32 | mixtral_bf16 | dsv3_bf16 | dsv3_fp8fp4 | "
                         "dsv3_fp8fp4_zipf | decode_fp8fp4 (default: the headline line plus the sweep)")
    ap.add_argument("--T", type=int, default=None, help="tokens of --workload (default: the workload's)")
    ap.add_argument("--path", choices=["best", "fused", "unfused"], default="best",
                    help="entry point to time (best: both, the faster gives the value)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB five times (the known-size "
                         "kernel that scales the HBM byte counters) and exit")
    ap.add_argument("--cpu-seconds", type=float, default=None, help="CPU-oracle sample budget (all cores)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--entry", choices=["capacity", "ep", "gemm"], default=None,
                    help="measure only the sweep entry of this kind (the capacity-factor layer, one EP "
                         "rank's share, the dense GEMM) and print its JSON")
    ap.add_argument("--flush-mb", type=int, default=None,
                    help="read this many MiB before each step to evict the 256 MB Infinity Cache and "
                         "the L2s (default: on for T <= 64)")
    return ap.parse_args(argv)


# ---- algorithmic work -----------------------------------------------------------------

def flops_of(w):
    experts = 6.0 * w.d * w.F * w.T * (w.k + w.S)
    router = 2.0 * w.T * w.d * w.E
    return experts, router


def weight_bytes_per_group(w):
    if w.mode == "fp8_mxfp4":
        return 2 * w.F * w.d // 2 + 2 * w.F * w.d // 32 + w.d * w.F // 2 + w.d * w.F // 32
    if w.mode == "fp8_fp8":
        return 3 * w.F * w.d + 3 * w.F * w.d // 128 * 4
    eb = 4 if w.mode == "f32" else 2
    return 3 * w.F * w.d * eb


def layer_bytes(w, counts):
    """Algorithmic bytes of a whole step: the touched groups' weights once, the router
    weights, x read and y written."""
    act = 4 if w.mode == "f32" else 2
    touched = int((np.asarray(counts) > 0).sum())
    return touched * weight_bytes_per_group(w) + w.E * w.d * act + 2 * w.T * w.d * act


def kernel_work(w, name, counts):
    """Algorithmic (flops, bytes) of one launch of a kernel, from the definitions:
    weights of the touched groups counted once, activations read once, outputs written once."""
    rows = w.T * (w.k + w.S)
    touched = int((np.asarray(counts) > 0).sum())
    act = 4 if w.mode == "f32" else 2
    if w.mode == "fp8_mxfp4":
        w1b = 2 * w.F * w.d // 2 + 2 * w.F * w.d // 32
        w2b = w.d * w.F // 2 + w.d * w.F // 32
        xb, hb = w.T * w.d * (1 + 4 / 128), rows * w.F * (1 + 4 / 128)
    elif w.mode == "fp8_fp8":
        w1b = 2 * w.F * w.d * (1 + 4 / 128)
        w2b = w.d * w.F * (1 + 4 / 128)
        xb, hb = w.T * w.d * (1 + 4 / 128), rows * w.F * (1 + 4 / 128)
    else:
        w1b, w2b = 2 * w.F * w.d * act, w.d * w.F * act
        xb, hb = w.T * w.d * act, rows * w.F * act
    if name == "linear1":
        return 4.0 * rows * w.F * w.d, touched * w1b + xb + hb
    if name == "linear2":
        return 2.0 * rows * w.F * w.d, touched * w2b + hb + rows * w.d * (4 if w.mode == "f32" else 2)
    if name == "route":
        return 2.0 * w.T * w.d * w.E, w.T * w.d * act + w.E * w.d * act + w.T * w.k * 8
    if name == "combine":
        return 2.0 * w.T * w.d * (w.k + w.S), rows * w.d * (4 if w.mode == "f32" else 2) + w.T * w.d * act
    if name in ("fused", "layer_fused"):
        f_e, f_r = flops_of(w)
        return f_e + f_r, layer_bytes(w, counts)
    return 0.0, 0.0


def load_stats(w, counts):
    """Per-expert load of the routed experts: max / mean, Gini coefficient, experts touched."""
    c = np.asarray(counts, dtype=np.float64)[: w.E]
    mean = c.mean()
    gini = float(np.abs(c[:, None] - c[None, :]).sum() / (2.0 * w.E * w.E * mean)) if mean > 0 else 0.0
    return {"max_over_mean": float(c.max() / mean) if mean > 0 else 0.0, "gini": gini,
            "max_rows": int(c.max()), "min_rows": int(c.min()), "experts_touched": int((c > 0).sum())}


def roofline_of(w, kernel, kms, counts):
    kf, kb = kernel_work(w, kernel, counts)
    peak_f = PEAK[w.mode]
    ridge = peak_f * 1e12 / (PEAK_HBM * 1e9)
    if w.mode == "f32":
        roof = {"bound": "alu", "achieved": kf / (kms * 1e-3) / 1e12, "peak": peak_f, "unit": "TFLOP/s"}
    elif kb > 0 and kf / kb < ridge:
        roof = {"bound": "hbm", "achieved": kb / (kms * 1e-3) / 1e9, "peak": PEAK_HBM, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": kf / (kms * 1e-3) / 1e12, "peak": peak_f, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_of(w, kernel)
    roof["traffic_unit"] = "bytes per launch"
    roof["kernel"] = kernel
    roof["launch_ms"] = kms
    roof["work_per_launch"] = {"flop": kf, "bytes": kb}
    return roof


# ---- counter traffic ----------------------------------------------------------------------

_COMMON = ("common.hpp", "dispatch_dev.hpp")
KERNEL_SOURCES = {
    ("linear1", "fp8_mxfp4"): ("ffn.hip", "ffn_fp8.hip", "gemm_fp8_dev.hpp") + _COMMON,
    ("linear2", "fp8_mxfp4"): ("ffn.hip", "ffn_fp8.hip", "gemm_fp8_dev.hpp") + _COMMON,
    ("linear1", "fp8_fp8"): ("ffn.hip", "ffn_fp8x8.hip", "gemm_fp8x8_dev.hpp", "gemm_fp8_dev.hpp") + _COMMON,
    ("linear2", "fp8_fp8"): ("ffn.hip", "ffn_fp8x8.hip", "gemm_fp8x8_dev.hpp", "gemm_fp8_dev.hpp") + _COMMON,
    ("linear1", "bf16"): ("ffn.hip", "gemm_bf16_dev.hpp") + _COMMON,
    ("linear2", "bf16"): ("ffn.hip", "gemm_bf16_dev.hpp") + _COMMON,
    ("combine", None): ("combine.hip", "combine_dev.hpp", "common.hpp"),
    ("gemm_fp8_mxfp4", None): ("ffn_fp8.hip", "gemm_fp8_dev.hpp", "common.hpp"),
    ("route", None): ("route.hip", "route_dev.hpp", "common.hpp"),
}


def sources_hash(kernel=None, mode=None) -> str:
    """Hash of the kernel sources a kernel is built from (all of csrc/*.hip and *.hpp when the
    kernel is not listed): hardware counters are valid for these sources only."""
    csrc = os.path.join(ROOT, "mixture_experts_layer_dispatch_amd", "csrc")
    names = KERNEL_SOURCES.get((kernel, mode)) or KERNEL_SOURCES.get((kernel, None))
    if names is None:
        names = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp")))
    h = hashlib.sha256()
    for f in sorted(names):
        path = os.path.join(csrc, f)
        h.update(f.encode())
        if os.path.exists(path):
            with open(path, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_of(w, kernel, label=None):
    """HBM bytes per launch of `kernel` on workload w (or the sweep entry `label`) from
    profiles/traffic.txt: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over the kernel's
    dispatches) each scaled by the ratio of known bytes to counter bytes for a plain copy.  None
    when absent or when the sources changed."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    cur = sources_hash(kernel, w.mode)
    name = label or w.name
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or "=" not in line:
                continue
            kv = dict(tok.split("=", 1) for tok in line.split() if "=" in tok)
            if kv.get("workload") == name and int(kv.get("T", -1)) == w.T and kv.get("kernel") == kernel:
                if kv.get("sources") != cur:
                    return None
                return (float(kv["fetch_kib"]) * float(kv["fetch_scale"]) +
                        float(kv["write_kib"]) * float(kv["write_scale"])) * 1024.0
    return None


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB five times (read {mib} MiB and write {mib} MiB per copy)")


# ---- inputs ---------------------------------------------------------------------------------

def upload(inp):
    import torch

    w = inp["workload"]

    def dev(a, kind):
        if a is None:
            return None
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    act = "f32" if w.mode == "f32" else "bf16"
    wk = "u8" if w.mode in FP8 else act
    return {"x": dev(inp["x"], act), "w_router": dev(inp["w_router"], act), "bias": dev(inp["bias"], "f32"),
            "w1": dev(inp["w1"], wk), "w2": dev(inp["w2"], wk), "w1_scale": dev(inp["w1_scale"], "u8"),
            "w2_scale": dev(inp["w2_scale"], "u8")}


class Inputs:
    """Host and device inputs of one weight set, generated at the largest T it serves; a
    smaller T takes the first T rows of x (element i of x is drawn from counter i, so the
    rows equal those drawn at that T).  Workloads that differ only in their router's gating
    and bias share the weights."""

    def __init__(self):
        self.key = None
        self.inp = None
        self.dev = None

    def get(self, w, T_max):
        import synth

        key = (w.seed, w.mode, w.d, w.E, w.F, w.S)
        if self.key != key or self.inp["x"].shape[0] < T_max:
            self.release()
            t0 = time.time()
            self.inp = synth.make_inputs(w.with_T(T_max))
            log(f"inputs for {w.name} (T={T_max}) generated on host in {time.time() - t0:.1f}s")
            self.dev = upload(self.inp)
            self.key = key
        import synth as _s
        inp = dict(self.inp, workload=w, x=self.inp["x"][: w.T], bias=_s.zipf_bias(w))
        dev = dict(self.dev, x=self.dev["x"][: w.T])
        if inp["bias"] is None:
            dev["bias"] = None
        else:
            import torch
            dev["bias"] = torch.from_numpy(inp["bias"]).cuda()
        return inp, dev

    def release(self):
        import torch

        self.inp = self.dev = self.key = None
        torch.cuda.empty_cache()


# ---- one layer entry ------------------------------------------------------------------------

def time_steps(step, steps, warmup, flush=None):
    """Warm-up, then exactly `steps` timed steps between synchronisations: the wall clock over
    them (mean) and each step's HIP-event time (median, p10, p90).  With `flush`, a cache flush
    runs before each step, outside its events, and the mean is taken over the events."""
    import torch

    for _ in range(warmup):
        if flush:
            flush()
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        if flush:
            flush()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = np.array([a.elapsed_time(b) for a, b in ev])
    mean = float(per.mean()) if flush else wall
    return {"mean": mean, "median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
            "p90": float(np.percentile(per, 90)), "events_mean": float(per.mean())}


def cpu_baseline(w, inp, seconds, seconds_1t):
    """The oracle (as it stands) on a bounded, evenly spaced token sample of the same layer,
    routing included: all host cores, then one thread."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    f_exp, f_rt = flops_of(w)
    per_tok = (f_exp + f_rt) / w.T

    def rate(threads, budget):
        n0 = min(w.T, threads)
        ta = time.perf_counter()
        oracle.layer(inp, tokens=np.linspace(0, w.T - 1, n0).astype(np.int64), nthreads=threads)
        t_probe = time.perf_counter() - ta
        n = int(min(w.T, max(n0, n0 * budget / max(t_probe, 1e-6))))
        toks = np.linspace(0, w.T - 1, n).astype(np.int64)
        ta = time.perf_counter()
        oracle.layer(inp, tokens=toks, nthreads=threads)
        dt = time.perf_counter() - ta
        return n, dt

    n, dt = rate(cores, seconds)
    n1, dt1 = rate(1, seconds_1t)
    return {"value": n / dt * per_tok / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "tokens_per_s": n / dt,
            "sample": f"{n} of {w.T} tokens (evenly spaced) through the full layer incl. routing, "
                      f"fp64 C oracle on {cores} threads, {dt:.1f}s",
            "one_thread": {"tokens_per_s": n1 / dt1, "value": n1 / dt1 * per_tok / 1e12, "unit": "TFLOP/s",
                           "sample": f"{n1} tokens on 1 thread, {dt1:.1f}s"}}


def measure_layer(w, inp, d, args, steps, warmup, cpu_s, cpu_1t):
    import torch

    import mixture_experts_layer_dispatch_amd as moe

    log(f"{w.name}: mode={w.mode} T={w.T} d={w.d} E={w.E} k={w.k} F={w.F} shared={w.S} {w.gating}")
    cfg = moe.Config(T=w.T, d=w.d, E=w.E, k=w.k, F=w.F, n_shared=w.S, gating=w.gating, mode=w.mode)
    ws = moe.alloc_workspace(cfg)
    y = torch.empty(w.T, w.d, dtype=moe.act_dtype(cfg), device="cuda")
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device="cuda")
    gate = torch.empty(w.T, w.k, dtype=torch.float32, device="cuda")
    counts = torch.empty(w.G, dtype=torch.int32, device="cuda")
    flush_mb = args.flush_mb if args.flush_mb is not None else (512 if w.T <= 64 else 0)
    flush_buf = torch.ones(flush_mb * (1 << 18), dtype=torch.float32, device="cuda") if flush_mb else None

    def flush():
        flush_buf.amax()  # a read-only sweep: evicts cached weights without dirty lines

    args_l = (cfg, d["x"], d["w_router"], d["w1"], d["w2"], d["w1_scale"], d["w2_scale"], d["bias"])

    def step_fused():
        moe.layer_fused(*args_l, ws=ws, y=y, topk_idx=idx, topk_gate=gate, counts=counts)

    def step_unfused():
        moe.layer_unfused(*args_l, ws=ws)

    steps_of = {"fused": step_fused, "unfused": step_unfused}
    timed = {}
    for name in (("fused", "unfused") if args.path == "best" else (args.path,)):
        timed[name] = time_steps(steps_of[name], steps, warmup, flush if flush_buf is not None else None)
        log(f"  {name}: mean {timed[name]['mean']:.4f} ms, median {timed[name]['median']:.4f} ms")
    assert moe.read_device_error(cfg, ws) == 0, "device error during the timed steps"
    path = min(timed, key=lambda n: timed[n]["mean"])
    t = timed[path]
    ms = t["mean"]

    # per-kernel timing: HIP events on each launch's stream, same steps
    moe.profile_report()
    moe.profile_enable(True)
    for _ in range(steps):
        if flush_buf is not None:
            flush()
        steps_of[path]()
    torch.cuda.synchronize()
    prof = moe.profile_report()
    moe.profile_enable(False)
    kernels = {n: {"launches_per_step": c / steps, "mean_ms": tt / c} for n, (c, tt) in prof.items()}
    log("  kernels: " + ", ".join(f"{n} {v['mean_ms']:.4f}ms" for n, v in kernels.items()))

    _, routing = moe.layer_unfused(*args_l, ws=ws)
    counts_np = routing["counts"].cpu().numpy()
    f_exp, f_rt = flops_of(w)
    alg_bytes = layer_bytes(w, counts_np)
    dom = max(kernels.items(), key=lambda kv: kv[1]["mean_ms"] * kv[1]["launches_per_step"])[0]
    out = {
        "workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "F": w.F, "n_shared": w.S,
        "gating": w.gating, "zipf_alpha": w.zipf_alpha, "dtype": DTYPE[w.mode], "path": path,
        "ms_per_step": ms, "ms_median": t["median"], "ms_p10": t["p10"], "ms_p90": t["p90"],
        "active_tflops": (f_exp + f_rt) / (ms * 1e-3) / 1e12,
        "tokens_per_s": w.T / (ms * 1e-3),
        "algorithmic_GBps": alg_bytes / (ms * 1e-3) / 1e9,
        "hbm_frac": alg_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM,
        "mfma_frac": (f_exp + f_rt) / (ms * 1e-3) / 1e12 / PEAK[w.mode],
        "active_tflop": {"experts": f_exp / 1e12, "router": f_rt / 1e12},
        "path_ms": {n: v["mean"] for n, v in timed.items()},
        "path_ms_median": {n: v["median"] for n, v in timed.items()},
        "fused_speedup_vs_unfused": (timed["unfused"]["mean"] / timed["fused"]["mean"]) if len(timed) == 2 else None,
        "load": load_stats(w, counts_np),
        "kernels": kernels,
        "roofline": roofline_of(w, dom, kernels[dom]["mean_ms"], counts_np),
        "timing": ("wall clock over the timed steps; median/p10/p90 from HIP events around each step"
                   if flush_buf is None else
                   f"HIP events around each step; {flush_mb} MiB read before each step to evict caches"),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, inp, cpu_s, cpu_1t)
        log(f"  cpu oracle: {out['cpu_baseline']['tokens_per_s']:.2f} tokens/s on "
            f"{out['cpu_baseline']['cores']} threads, {out['cpu_baseline']['one_thread']['tokens_per_s']:.2f} on one")
    else:
        out["cpu_baseline"] = None
    del ws, flush_buf
    return out


def kernel_times(step, steps):
    """Per-kernel mean durations (HIP events on each launch's own stream) over `steps` steps."""
    import torch

    import mixture_experts_layer_dispatch_amd as moe

    moe.profile_report()
    moe.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = moe.profile_report()
    moe.profile_enable(False)
    return {n: {"launches_per_step": c / steps, "mean_ms": tt / c} for n, (c, tt) in prof.items()}


def roofline_flops(kf, kb, mode, kernel, kms, w=None, label=None):
    peak_f = PEAK[mode]
    ridge = peak_f * 1e12 / (PEAK_HBM * 1e9)
    if kb > 0 and kf / kb < ridge:
        roof = {"bound": "hbm", "achieved": kb / (kms * 1e-3) / 1e9, "peak": PEAK_HBM, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": kf / (kms * 1e-3) / 1e12, "peak": peak_f, "unit": "TFLOP/s"}
    traffic = traffic_of(w, kernel, label) if w is not None else None
    roof.update({"frac": roof["achieved"] / roof["peak"], "traffic": traffic, "traffic_unit": "bytes per launch",
                 "kernel": kernel, "launch_ms": kms, "work_per_launch": {"flop": kf, "bytes": kb}})
    return roof


def measure_capacity(w, inp, d, args, steps, warmup, factor, cpu_s, cpu_1t):
    """The layer with the capacity-factor dispatch (route -> dispatch_capacity -> ffn -> combine):
    each routed expert takes at most floor(factor * T * k / E) slots.  Also times one
    aux-loss-free bias update from the step's counts."""
    import torch

    import mixture_experts_layer_dispatch_amd as moe
    import oracle

    cfg = moe.Config(T=w.T, d=w.d, E=w.E, k=w.k, F=w.F, n_shared=w.S, gating=w.gating, mode=w.mode)
    cap = moe.capacity_of(factor, cfg)
    log(f"{w.name} with capacity factor {factor}: {cap} slots per expert, T={w.T}")
    ws = moe.alloc_workspace(cfg)
    fp8 = w.mode in FP8
    # every output allocated once, as a serving loop would: the timed steps launch kernels only
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device="cuda")
    gate = torch.empty(w.T, w.k, dtype=torch.float32, device="cuda")
    dsp = moe.dispatch_capacity(cfg, moe.route(cfg, d["x"], d["w_router"], d["bias"], ws=ws, topk_idx=idx,
                                               topk_gate=gate)[0], cap, d["x"] if fp8 else None, ws=ws)
    yp = torch.empty(cfg.rows, w.d, dtype=torch.float32 if w.mode == "f32" else torch.bfloat16, device="cuda")
    y = torch.empty(w.T, w.d, dtype=moe.act_dtype(cfg), device="cuda")
    state = {"idx": idx, "gate": gate, "dsp": dsp, "y": y}

    def step():
        moe.route(cfg, d["x"], d["w_router"], d["bias"], ws=ws, topk_idx=idx, topk_gate=gate)
        moe.dispatch_capacity(cfg, idx, cap, d["x"] if fp8 else None, ws=ws, out=dsp)
        moe.ffn(cfg, d["w1"], d["w2"], d["w1_scale"], d["w2_scale"], x=None if fp8 else d["x"], xq=dsp["xq"],
                xq_scale=dsp["xq_scale"], offsets=dsp["offsets"], row_to_slot=dsp["row_to_slot"], ws=ws, y_perm=yp)
        moe.combine(cfg, yp, dsp["slot_to_row"], gate, y=y)

    t = time_steps(step, steps, warmup)
    assert moe.read_device_error(cfg, ws) == 0
    kernels = kernel_times(step, steps)
    dsp = state["dsp"]
    kept = dsp["counts"].cpu().numpy()
    dropped = dsp["dropped"].cpu().numpy()
    raw = kept[: w.E] + dropped
    # one bias update from the load the router asked for (kept + dropped)
    bias = torch.zeros(w.E, dtype=torch.float32, device="cuda")
    load = torch.from_numpy(raw.astype(np.int32)).cuda()
    tb = time_steps(lambda: moe.bias_update(cfg, load, bias, 1e-3), steps, warmup)
    ms = t["mean"]
    rows_kept = int(kept.sum())
    f_exp = 6.0 * w.d * w.F * rows_kept
    f_rt = 2.0 * w.T * w.d * w.E
    dom = max(kernels.items(), key=lambda kv: kv[1]["mean_ms"] * kv[1]["launches_per_step"])[0]
    kf = (4.0 if dom == "linear1" else 2.0) * rows_kept * w.F * w.d
    kb = kernel_work(w, dom, kept)[1]
    out = {
        "kind": "capacity", "workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "F": w.F, "n_shared": w.S,
        "gating": w.gating, "zipf_alpha": w.zipf_alpha, "dtype": DTYPE[w.mode], "path": "unfused",
        "capacity_factor": factor, "capacity": cap, "dropped_slots": int(dropped.sum()),
        "dropped_frac": float(dropped.sum()) / (w.T * w.k), "experts_over_capacity": int((dropped > 0).sum()),
        "ms_per_step": ms, "ms_median": t["median"], "ms_p10": t["p10"], "ms_p90": t["p90"],
        "active_tflops": (f_exp + f_rt) / (ms * 1e-3) / 1e12, "tokens_per_s": w.T / (ms * 1e-3),
        "load": load_stats(w, raw), "kernels": kernels, "bias_update_ms": tb["median"],
        "roofline": roofline_flops(kf, kb, w.mode, dom, kernels[dom]["mean_ms"], w, f"{w.name}+capacity"),
        "timing": "wall clock over the timed steps; median/p10/p90 from HIP events around each step",
    }
    if not args.no_cpu:
        keep = (dsp["slot_to_row"].cpu().numpy() >= 0).reshape(w.T, w.k)
        idx, gate = state["idx"].cpu().numpy(), state["gate"].cpu().numpy()
        cores = len(os.sched_getaffinity(0))
        per_tok = (f_exp + f_rt) / w.T

        def rate(threads, budget):
            n0 = min(w.T, threads)
            ta = time.perf_counter()
            oracle.layer_dropping(inp, idx, gate, keep, tokens=np.arange(n0), nthreads=threads)
            tp = time.perf_counter() - ta
            n = int(min(w.T, max(n0, n0 * budget / max(tp, 1e-6))))
            toks = np.linspace(0, w.T - 1, n).astype(np.int64)
            ta = time.perf_counter()
            oracle.layer_dropping(inp, idx, gate, keep, tokens=toks, nthreads=threads)
            return n, time.perf_counter() - ta

        n, dt = rate(cores, cpu_s)
        n1, dt1 = rate(1, cpu_1t)
        out["cpu_baseline"] = {"value": n / dt * per_tok / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                               "tokens_per_s": n / dt,
                               "sample": f"{n} of {w.T} tokens (evenly spaced) through the experts with the GPU's "
                                         f"routing and drops, fp64 C oracle on {cores} threads, {dt:.1f}s",
                               "one_thread": {"tokens_per_s": n1 / dt1, "value": n1 / dt1 * per_tok / 1e12,
                                              "unit": "TFLOP/s", "sample": f"{n1} tokens on 1 thread, {dt1:.1f}s"}}
    else:
        out["cpu_baseline"] = None
    log(f"  capacity: {ms:.4f} ms, dropped {out['dropped_slots']} of {w.T * w.k} slots, bias update "
        f"{tb['median'] * 1e3:.1f} us")
    return out


def ep_receive(w, E_local, n_src, seed=7000):
    """Counts and rows of one expert-parallel rank: n_src ranks of w.T tokens each route
    uniformly over w.E experts (top-k), this rank owning experts 0 .. E_local - 1; the rows are
    seeded FP8 rows (the wire format: e4m3 codes with power-of-two scales per 128)."""
    import synth

    rng = np.random.default_rng(seed)
    counts = np.zeros((E_local, n_src), dtype=np.int32)
    for q in range(n_src):
        choice = np.argpartition(rng.random((w.T, w.E)), w.k, axis=1)[:, : w.k]
        counts[:, q] = np.bincount(choice.reshape(-1), minlength=w.E)[:E_local]
    R = int(counts.sum())
    rq, rs = synth.fp8_rows(seed, 21, R, w.d, 1.0)
    xq, xs = synth.fp8_rows(seed, 22, w.T, w.d, 1.0)
    return counts, (rq, rs), (xq, xs)


def measure_ep(w, inp, d, args, steps, warmup, E_local, n_src, cpu_s, cpu_1t):
    """One expert-parallel rank's share at its real shape: E_local local experts (and the
    shared one) over the rows n_src ranks of w.T tokens send it, plus its own w.T tokens."""
    import torch

    import mixture_experts_layer_dispatch_amd as moe
    import oracle

    counts, recv, own = ep_receive(w, E_local, n_src)
    R = int(counts.sum())
    log(f"EP rank: {E_local} local experts + shared, {n_src} sources x {w.T} tokens -> {R} received rows")
    G = w.E + w.S
    sel = torch.tensor(list(range(E_local)) + [w.E], device="cuda")  # local experts, then the shared one
    w1, w2, w1s, w2s = (d[k].index_select(0, sel).contiguous() for k in ("w1", "w2", "w1_scale", "w2_scale"))
    cfg = moe.Config(T=w.T, d=w.d, E=E_local, k=1, F=w.F, n_shared=w.S, mode=w.mode)
    ws = moe.ep_workspace(cfg, R)
    rc = torch.from_numpy(counts).cuda()
    rq, rs = torch.from_numpy(recv[0]).cuda(), torch.from_numpy(recv[1]).cuda()
    xq, xs = torch.from_numpy(own[0]).cuda(), torch.from_numpy(own[1]).cuda()
    yr = torch.empty(R, w.d, dtype=torch.bfloat16, device="cuda")
    ysh = torch.empty(w.T, w.d, dtype=torch.bfloat16, device="cuda")

    def step():
        moe.ep_ffn(cfg, w1, w2, w1s, w2s, recv_counts=rc, recv_xq=rq, recv_xs=rs, xq=xq, xs=xs, ws=ws, y_recv=yr,
                   y_shared=ysh)

    t = time_steps(step, steps, warmup)
    assert moe.read_device_error(cfg, ws) == 0
    kernels = kernel_times(step, steps)
    ms = t["mean"]
    rows = R + w.S * w.T
    flop = 6.0 * w.d * w.F * rows
    wbytes = (E_local + w.S) * weight_bytes_per_group(w)
    dom = "linear1"
    kf = 4.0 * R * w.F * w.d
    kb = E_local * (weight_bytes_per_group(w) * 2 // 3) + R * w.d * (1 + 4 / 128) + R * w.F * (1 + 4 / 128)
    out = {
        "kind": "ep", "workload": w.name, "T": w.T, "d": w.d, "E_local": E_local, "n_src": n_src, "F": w.F,
        "n_shared": w.S, "received_rows": R, "dtype": DTYPE[w.mode], "path": "moe_ep_ffn",
        "ms_per_step": ms, "ms_median": t["median"], "ms_p10": t["p10"], "ms_p90": t["p90"],
        "active_tflops": flop / (ms * 1e-3) / 1e12, "rows_per_s": rows / (ms * 1e-3),
        "algorithmic_GBps": (wbytes + rows * w.d * (1 + 4 / 128) + rows * w.d * 2) / (ms * 1e-3) / 1e9,
        "mfma_frac": flop / (ms * 1e-3) / 1e12 / PEAK[w.mode], "kernels": kernels,
        "load": {"rows_per_expert_max": int(counts.sum(1).max()), "rows_per_expert_min": int(counts.sum(1).min())},
        "roofline": roofline_flops(kf, kb, w.mode, dom, kernels[dom]["mean_ms"], w, f"{w.name}+ep"),
        "timing": "wall clock over the timed steps; median/p10/p90 from HIP events around each step",
    }
    if not args.no_cpu:
        ex = {"workload": w, "w1": inp["w1"][list(range(E_local)) + [w.E]], "w2": inp["w2"][list(range(E_local)) + [w.E]],
              "w1_scale": inp["w1_scale"][list(range(E_local)) + [w.E]],
              "w2_scale": inp["w2_scale"][list(range(E_local)) + [w.E]]}
        import synth as _s
        ex["workload"] = _s.Workload("ep", w.seed, w.mode, w.T, w.d, E_local, 1, w.F, w.S, "softmax")
        offs = np.concatenate([[0], np.cumsum(counts.sum(axis=1))])
        cores = len(os.sched_getaffinity(0))

        def rate(threads, budget):
            from concurrent.futures import ThreadPoolExecutor

            def run(rws):
                def one(r):
                    g = int(np.searchsorted(offs, r, side="right") - 1)
                    xin = oracle.dequant_e4m3_rows(recv[0][r:r + 1], recv[1][r:r + 1])
                    oracle.expert_rows(ex, g, xin)
                with ThreadPoolExecutor(max_workers=threads) as pool:
                    list(pool.map(one, rws))

            n0 = threads
            ta = time.perf_counter()
            run(np.linspace(0, R - 1, n0).astype(np.int64))
            tp = time.perf_counter() - ta
            n = int(min(R, max(n0, n0 * budget / max(tp, 1e-6))))
            ta = time.perf_counter()
            run(np.linspace(0, R - 1, n).astype(np.int64))
            return n, time.perf_counter() - ta

        n, dt = rate(cores, cpu_s)
        n1, dt1 = rate(1, cpu_1t)
        per_row = 6.0 * w.d * w.F
        out["cpu_baseline"] = {"value": n / dt * per_row / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                               "rows_per_s": n / dt,
                               "sample": f"{n} of {R} received rows (evenly spaced) through their expert, fp64 C "
                                         f"oracle on {cores} threads, {dt:.1f}s",
                               "one_thread": {"rows_per_s": n1 / dt1, "value": n1 / dt1 * per_row / 1e12,
                                              "unit": "TFLOP/s", "sample": f"{n1} rows on 1 thread, {dt1:.1f}s"}}
    else:
        out["cpu_baseline"] = None
    log(f"  EP rank: {ms:.4f} ms, {out['active_tflops']:.0f} TFLOP/s")
    return out


def measure_gemm(w, inp, d, args, steps, warmup, M, N, K, cpu_s, cpu_1t):
    """The dense FP8 x MXFP4 GEMM: A [M, K] seeded FP8 rows, B the first N rows of the layer's
    (shared expert's) W1 -- an [N, K] MXFP4 matrix."""
    import torch

    import mixture_experts_layer_dispatch_amd as moe
    import oracle
    import synth

    log(f"dense FP8 x MXFP4 GEMM: M={M} N={N} K={K}")
    a, a_s = synth.fp8_rows(7100, 31, M, K, 1.0)
    b = d["w1"][w.E][:N].contiguous()
    b_s = d["w1_scale"][w.E][:N].contiguous()
    ad, asd = torch.from_numpy(a).cuda(), torch.from_numpy(a_s).cuda()
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.GEMM_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")

    def step():
        moe.gemm_fp8_mxfp4(ad, asd, b, b_s, ws=ws, c=c)

    t = time_steps(step, steps, warmup)
    kernels = kernel_times(step, steps)
    ms = t["mean"]
    flop = 2.0 * M * N * K
    kb = N * K // 2 + N * K // 32 + M * K * (1 + 4 / 128) + M * N * 2
    out = {
        "kind": "gemm", "M": M, "N": N, "K": K, "dtype": "fp8e4m3 x mxfp4", "path": "moe_gemm_fp8_mxfp4",
        "ms_per_step": ms, "ms_median": t["median"], "ms_p10": t["p10"], "ms_p90": t["p90"],
        "tflops": flop / (ms * 1e-3) / 1e12, "mfma_frac": flop / (ms * 1e-3) / 1e12 / PEAK["fp8_mxfp4"],
        "kernels": kernels,
        "roofline": roofline_flops(flop, kb, "fp8_mxfp4", "gemm_fp8_mxfp4", kernels["gemm_fp8_mxfp4"]["mean_ms"],
                                   w.with_T(M), f"gemm_{M}x{N}x{K}"),
        "timing": "wall clock over the timed steps; median/p10/p90 from HIP events around each step",
    }
    if not args.no_cpu:
        bh, bsh = inp["w1"][w.E][:N], inp["w1_scale"][w.E][:N]
        cores = len(os.sched_getaffinity(0))

        def rate(threads, budget):
            from concurrent.futures import ThreadPoolExecutor

            def run(rws):
                with ThreadPoolExecutor(max_workers=threads) as pool:
                    list(pool.map(lambda r: oracle.gemm_fp8_mxfp4(a, a_s, bh, bsh, rows=[r]), rws))

            n0 = threads
            ta = time.perf_counter()
            run(np.linspace(0, M - 1, n0).astype(np.int64))
            tp = time.perf_counter() - ta
            n = int(min(M, max(n0, n0 * budget / max(tp, 1e-6))))
            ta = time.perf_counter()
            run(np.linspace(0, M - 1, n).astype(np.int64))
            return n, time.perf_counter() - ta

        n, dt = rate(cores, cpu_s)
        n1, dt1 = rate(1, cpu_1t)
        per_row = 2.0 * N * K
        out["cpu_baseline"] = {"value": n / dt * per_row / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                               "rows_per_s": n / dt,
                               "sample": f"{n} of {M} rows of C, fp64 C oracle on {cores} threads, {dt:.1f}s",
                               "one_thread": {"rows_per_s": n1 / dt1, "value": n1 / dt1 * per_row / 1e12,
                                              "unit": "TFLOP/s", "sample": f"{n1} rows on 1 thread, {dt1:.1f}s"}}
    else:
        out["cpu_baseline"] = None
    log(f"  dense GEMM: {ms:.4f} ms, {out['tflops']:.0f} TFLOP/s")
    return out


def line_of(e, args, sweep=None):
    """The JSON line of the headline entry e."""
    decode = e["T"] == 1
    out = {
        "metric": METRIC,
        "value": e["active_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": e["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": e["dtype"],
        "data": "synthetic (seeded Philox4x32-10 normals; random-init weights of the workload's shape)",
        "config": {"workload": e["workload"], "T": e["T"], "d": e["d"], "E": e["E"], "k": e["k"], "F": e["F"],
                   "n_shared": e["n_shared"], "gating": e["gating"], "zipf_alpha": e["zipf_alpha"],
                   "path": e["path"], "timing": e["timing"]},
        "roofline": e["roofline"],
        "cpu_baseline": e["cpu_baseline"],
    }
    if decode:
        out["GBps"] = e["algorithmic_GBps"]
    for key in ("ms_median", "ms_p10", "ms_p90", "tokens_per_s", "algorithmic_GBps", "hbm_frac", "mfma_frac",
                "active_tflop", "path_ms", "path_ms_median", "fused_speedup_vs_unfused", "load", "kernels"):
        out[key] = e[key]
    if sweep is not None:
        out["sweep"] = sweep
    return out


def main(argv=None):
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr, flush=True)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    t_start = time.time()
    cache = Inputs()

    if args.workload is not None:
        w = synth.WORKLOADS[args.workload]
        if args.T is not None:
            w = w.with_T(args.T)
        elif w.t_values:
            w = w.with_T(w.t_values[0] if args.workload.startswith("decode") else 8192)
        inp, d = cache.get(w, w.T)
        cpu_s = args.cpu_seconds if args.cpu_seconds is not None else 12.0
        e = measure_layer(w, inp, d, args, args.steps, args.warmup, cpu_s, cpu_s / 3)
        print(json.dumps(line_of(e, args)), flush=True)
        return

    # the default run: the headline entry, then the sweep (entries sharing weights together);
    # --entry: that one entry alone
    sweep = [e for e in SWEEP if e["kind"] == args.entry] if args.entry else SWEEP
    t_max = {}
    for ent in sweep:
        key = synth.WORKLOADS[ent["workload"]].seed
        t_max[key] = max(t_max.get(key, 0), ent.get("T", 1))
    entries = []
    for ent in sweep:
        kind = ent["kind"]
        w = synth.WORKLOADS[ent["workload"]].with_T(ent.get("T", 1))
        inp, d = cache.get(w, t_max[w.seed])
        headline = (kind, ent["workload"], ent.get("T")) == HEADLINE
        steps = args.steps if headline else min(args.steps, 20)
        warmup = args.warmup if headline else min(args.warmup, 5)
        cpu_s, cpu_1t = ent["cpu"], ent["cpu1"]
        if args.cpu_seconds is not None:
            cpu_s = args.cpu_seconds if headline else min(cpu_s, args.cpu_seconds)
        if kind == "layer":
            e = measure_layer(w, inp, d, args, steps, warmup, cpu_s, cpu_1t)
            e["kind"] = "layer"
        elif kind == "capacity":
            e = measure_capacity(w, inp, d, args, steps, warmup, ent["factor"], cpu_s, cpu_1t)
        elif kind == "ep":
            e = measure_ep(w, inp, d, args, steps, warmup, ent["E_local"], ent["n_src"], cpu_s, cpu_1t)
        else:
            e = measure_gemm(w, inp, d, args, steps, warmup, ent["M"], ent["N"], ent["K"], cpu_s, cpu_1t)
        e["headline"] = headline
        entries.append(e)
        log(f"  done ({time.time() - t_start:.0f}s since start)")
    cache.release()
    if args.entry:
        print(json.dumps(entries[0]), flush=True)
        return
    head = next(e for e in entries if e["headline"])
    sweep = [e for e in entries if e is not head]
    print(json.dumps(line_of(head, args, sweep)), flush=True)


if __name__ == "__main__":
    main()
