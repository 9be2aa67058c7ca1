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
FP8 x MXFP4 layer at T = 512 and 8192 (and at 8192 with the sigmoid + Zipf-bias router),
and decode at T = 1 and 64 (whose metric is HBM GB/s).  Every entry carries its own
median / p10 / p90 step time, roofline of the dominant kernel, per-expert load
statistics and CPU-oracle rate (all host cores and one thread).

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

PEAK = {"bf16": 2500.0, "fp8_mxfp4": 5000.0, "f32": 157.3}  # dense TFLOP/s (MI355X spec)
PEAK_HBM = 8000.0  # GB/s
METRIC = "MoE-layer active TFLOPS & tokens/s at T=1..32768 (bf16, FP8×FP4); GB/s at T=1"
DTYPE = {"f32": "f32", "bf16": "bf16", "fp8_mxfp4": "fp8e4m3 x mxfp4"}

# (workload, T, CPU-oracle seconds on all cores, on one thread) of the default run, in
# execution order: entries that share weights run together.  The first is the headline.
HEADLINE = ("dsv3_fp8fp4", 32768)
SWEEP = [
    ("dsv3_fp8fp4", 32768, 12.0, 4.0),
    ("dsv3_fp8fp4", 8192, 4.0, 2.0),
    ("dsv3_fp8fp4", 512, 4.0, 2.0),
    ("dsv3_fp8fp4_zipf", 8192, 4.0, 2.0),
    ("decode_fp8fp4", 1, 2.0, 1.0),
    ("decode_fp8fp4", 64, 4.0, 2.0),
    ("dsv3_bf16", 8192, 4.0, 2.0),
    ("mixtral_bf16", 4096, 4.0, 2.0),
    ("tiny_f32", 64, 2.0, 1.0),
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
    ("linear1", "bf16"): ("ffn.hip", "gemm_bf16_dev.hpp") + _COMMON,
    ("linear2", "bf16"): ("ffn.hip", "gemm_bf16_dev.hpp") + _COMMON,
    ("combine", None): ("combine.hip", "combine_dev.hpp", "common.hpp"),
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


def traffic_of(w, kernel):
    """HBM bytes per launch of `kernel` on workload w from profiles/traffic.txt: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, mean over the kernel's dispatches) each scaled by the ratio of
    known bytes to counter bytes for a plain copy.  None when absent or when the sources changed."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    cur = sources_hash(kernel, w.mode)
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or "=" not in line:
                continue
            kv = dict(tok.split("=", 1) for tok in line.split() if "=" in tok)
            if kv.get("workload") == w.name and int(kv.get("T", -1)) == w.T and kv.get("kernel") == kernel:
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
    wk = "u8" if w.mode == "fp8_mxfp4" else act
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

    # the default run: the headline entry, then the sweep (entries sharing weights together)
    t_max = {}
    for name, T, _, _ in SWEEP:
        key = synth.WORKLOADS[name].seed
        t_max[key] = max(t_max.get(key, 0), T)
    entries = []
    for name, T, cpu_s, cpu_1t in SWEEP:
        w = synth.WORKLOADS[name].with_T(T)
        inp, d = cache.get(w, t_max[w.seed])
        headline = (name, T) == HEADLINE
        steps = args.steps if headline else min(args.steps, 20)
        warmup = args.warmup if headline else min(args.warmup, 5)
        if args.cpu_seconds is not None:
            cpu_s = args.cpu_seconds if headline else min(cpu_s, args.cpu_seconds)
        entries.append(measure_layer(w, inp, d, args, steps, warmup, cpu_s, cpu_1t))
        log(f"  done ({time.time() - t_start:.0f}s since start)")
    cache.release()
    head = next(e for e in entries if (e["workload"], e["T"]) == HEADLINE)
    sweep = [e for e in entries if e is not head]
    print(json.dumps(line_of(head, args, sweep)), flush=True)


if __name__ == "__main__":
    main()
