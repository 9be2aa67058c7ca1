#!/usr/bin/env python3
"""MoE-layer forward benchmark on one MI355X.

A step is one forward pass of the whole layer -- router, top-k, gates, dispatch,
linear1 + SwiGLU, linear2 and the gate-weighted combine -- over one batch of
seeded synthetic tokens with random-init weights of the workload's shape, all
resident in HBM before timing starts.  The default workload is the
Mixtral-shaped bf16 layer (T=4096, d=4096, E=8, k=2, F=14336).

Both entry points compute the same layer: the persistent single-launch kernel
(moe_layer_fused) and the chain of step kernels (route, dispatch, ffn, combine).  By
default both are timed and the faster one gives the reported value; the JSON names it
and carries both times.

Prints one JSON line: whole-layer active TFLOP/s (value), tokens/s, the roofline
of the dominant kernel (its algorithmic work over its mean duration, measured with
HIP events on its own stream during a timed pass), and the CPU oracle's rate on a
bounded token sample (cpu_baseline).  roofline.traffic is the HBM traffic of that
kernel from hardware counters (profiles/traffic.txt), reported only while the kernel
sources still hash to the ones the counters were taken with.
"""
from __future__ import annotations

import argparse
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


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_bf16",
                    help="tiny_f32 | mixtral_bf16 | dsv3_bf16 | dsv3_fp8fp4 | decode_fp8fp4")
    ap.add_argument("--T", type=int, default=None, help="tokens (default: the workload's)")
    ap.add_argument("--path", choices=["best", "fused", "unfused"], default="best",
                    help="entry point to report (best: time both, report the faster)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB five times (the known-size "
                         "kernel that scales the HBM byte counters) and exit")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-oracle sample budget")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--flush-mb", type=int, default=None,
                    help="read this many MiB between steps to evict the 256 MB Infinity Cache and "
                         "the L2s (default: on for T <= 64)")
    return ap.parse_args()


def flops_of(w):
    experts = 6.0 * w.d * w.F * w.T * (w.k + w.S)
    router = 2.0 * w.T * w.d * w.E
    return experts, router


def weight_bytes_per_group(w):
    if w.mode == "fp8_mxfp4":
        return 2 * w.F * w.d // 2 + 2 * w.F * w.d // 32 + w.d * w.F // 2 + w.d * w.F // 32
    eb = 4 if w.mode == "f32" else 2
    return 3 * w.F * w.d * eb


def kernel_work(w, name, counts):
    """Algorithmic (flops, bytes) of one launch of a kernel, from the definitions:
    weights of the touched groups counted once, activations read once, outputs written once."""
    rows = w.T * (w.k + w.S)
    touched = int((counts > 0).sum())
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
        return f_e + f_r, touched * (w1b + w2b) + w.E * w.d * act + 2 * w.T * w.d * act
    return 0.0, 0.0


def sources_hash() -> str:
    """Hash of the kernel sources, csrc/*.hip and *.hpp (hardware counters are valid for these only)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_dispatch_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".hpp")))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_of(w, kernel):
    """HBM bytes per launch of `kernel` on workload w from profiles/traffic.txt: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, mean over the kernel's dispatches) each scaled by the ratio of
    known bytes to counter bytes for a plain copy.  None when absent or when the sources changed."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    cur = sources_hash()
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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr, flush=True)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    import mixture_experts_layer_dispatch_amd as moe
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    if args.T is not None:
        w = w.with_T(args.T)
    elif w.t_values:
        w = w.with_T(w.t_values[0] if args.workload.startswith("decode") else 8192)
    log(f"workload {w.name}: mode={w.mode} T={w.T} d={w.d} E={w.E} k={w.k} F={w.F} shared={w.S} {w.gating}")
    t0 = time.time()
    inp = synth.make_inputs(w)
    log(f"inputs generated on host in {time.time() - t0:.1f}s")

    def dev(a, kind):
        if a is None:
            return None
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    act = "f32" if w.mode == "f32" else "bf16"
    wk = "u8" if w.mode == "fp8_mxfp4" else act
    x, wr, bias = dev(inp["x"], act), dev(inp["w_router"], act), dev(inp["bias"], "f32")
    w1, w2 = dev(inp["w1"], wk), dev(inp["w2"], wk)
    w1s, w2s = dev(inp["w1_scale"], "u8"), dev(inp["w2_scale"], "u8")
    cfg = moe.Config(T=w.T, d=w.d, E=w.E, k=w.k, F=w.F, n_shared=w.S, gating=w.gating, mode=w.mode)
    ws = moe.alloc_workspace(cfg)
    y = torch.empty(w.T, w.d, dtype=moe.act_dtype(cfg), device="cuda")
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device="cuda")
    gate = torch.empty(w.T, w.k, dtype=torch.float32, device="cuda")
    counts = torch.empty(w.G, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.time() - t0:.1f}s)")

    flush_mb = args.flush_mb if args.flush_mb is not None else (512 if w.T <= 64 else 0)
    flush_buf = torch.ones(flush_mb * (1 << 18), dtype=torch.float32, device="cuda") if flush_mb else None

    def flush():
        # a read-only sweep: evicts cached weights without leaving dirty lines to write back
        flush_buf.amax()  # fp32 max: one read pass, no widening copy

    def step_fused():
        moe.layer_fused(cfg, x, wr, w1, w2, w1s, w2s, bias, ws=ws, y=y, topk_idx=idx, topk_gate=gate,
                        counts=counts)

    def step_unfused():
        moe.layer_unfused(cfg, x, wr, w1, w2, w1s, w2s, bias, ws=ws)

    steps_of = {"fused": step_fused, "unfused": step_unfused}

    def time_path(step):
        """Warm-up, then exactly args.steps timed steps bracketed by synchronisations."""
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        assert moe.read_device_error(cfg, ws) == 0, "device error during warm-up"
        if flush_buf is None:
            torch.cuda.synchronize()
            ts = time.perf_counter()
            for _ in range(args.steps):
                step()
            torch.cuda.synchronize()
            return (time.perf_counter() - ts) * 1e3 / args.steps
        # a cache flush runs between steps, so each step is timed alone on the stream
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in ev:
            flush()
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    # ---- timed region(s) --------------------------------------------------------------
    timed = {}
    for name in (("fused", "unfused") if args.path == "best" else (args.path,)):
        timed[name] = time_path(steps_of[name])
        log(f"{name} step: {timed[name]:.4f} ms")
    path = min(timed, key=timed.get)
    ms = timed[path]
    step = steps_of[path]
    timing = ("wall clock over the timed steps" if flush_buf is None else
              f"HIP events around each step; {flush_mb} MiB read between steps to evict caches")
    assert moe.read_device_error(cfg, ws) == 0, "device error during the timed steps"

    # ---- per-kernel timing (HIP events on the launch stream, same steps) ------------------
    moe.profile_report()
    moe.profile_enable(True)
    for _ in range(args.steps):
        if flush_buf is not None:
            flush()
        step()
    torch.cuda.synchronize()
    prof = moe.profile_report()
    moe.profile_enable(False)
    kernels = {n: {"launches_per_step": c / args.steps, "mean_ms": t / c} for n, (c, t) in prof.items()}
    log("kernels: " + ", ".join(f"{n} {v['mean_ms']:.4f}ms" for n, v in kernels.items()))

    if "fused" in timed:
        counts_np = counts.cpu().numpy()  # written by the persistent kernel's steps
    else:  # one more (untimed) unfused step for the per-group row counts
        _, routing = moe.layer_unfused(cfg, x, wr, w1, w2, w1s, w2s, bias, ws=ws)
        counts_np = routing["counts"].cpu().numpy()
    f_exp, f_rt = flops_of(w)
    tflops = (f_exp + f_rt) / (ms * 1e-3) / 1e12
    tok_s = w.T / (ms * 1e-3)
    touched = int((counts_np > 0).sum())
    alg_bytes = touched * weight_bytes_per_group(w) + w.E * w.d * (4 if w.mode == "f32" else 2) + \
        2 * w.T * w.d * (4 if w.mode == "f32" else 2)
    gbs = alg_bytes / (ms * 1e-3) / 1e9

    # dominant kernel: the largest share of step time
    dom = max(kernels.items(), key=lambda kv: kv[1]["mean_ms"] * kv[1]["launches_per_step"])[0]
    kf, kb = kernel_work(w, dom, counts_np)
    kms = kernels[dom]["mean_ms"]
    peak_f = PEAK[w.mode]
    ridge = peak_f * 1e12 / (PEAK_HBM * 1e9)
    if w.mode == "f32":
        roof = {"bound": "alu", "achieved": kf / (kms * 1e-3) / 1e12, "peak": peak_f, "unit": "TFLOP/s"}
    elif kb > 0 and kf / kb < ridge:
        roof = {"bound": "hbm", "achieved": kb / (kms * 1e-3) / 1e9, "peak": PEAK_HBM, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": kf / (kms * 1e-3) / 1e12, "peak": peak_f, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    tr = traffic_of(w, dom)
    roof["traffic"] = tr
    roof["traffic_unit"] = "bytes per launch"
    roof["kernel"] = dom
    roof["work_per_launch"] = {"flop": kf, "bytes": kb}

    # ---- CPU oracle baseline (bounded sample) ------------------------------------------
    cpu = None
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        n0 = min(w.T, cores)
        ta = time.perf_counter()
        oracle.layer(inp, tokens=np.arange(n0), nthreads=cores)
        t_probe = time.perf_counter() - ta
        n = int(min(w.T, max(n0, n0 * args.cpu_seconds / max(t_probe, 1e-6))))
        toks = np.linspace(0, w.T - 1, n).astype(np.int64)
        ta = time.perf_counter()
        oracle.layer(inp, tokens=toks, nthreads=cores)
        t_cpu = time.perf_counter() - ta
        cpu_tok_s = n / t_cpu
        per_tok_flop = (f_exp + f_rt) / w.T
        cpu = {"value": cpu_tok_s * per_tok_flop / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "tokens_per_s": cpu_tok_s,
               "sample": f"{n} of {w.T} tokens (evenly spaced) through the full layer incl. routing, "
                         f"fp64 C oracle on {cores} threads, {t_cpu:.1f}s"}
        log(f"cpu oracle: {cpu_tok_s:.2f} tokens/s on {cores} threads")

    out = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8_mxfp4": "fp8e4m3 x mxfp4"}[w.mode],
        "data": "synthetic (seeded Philox4x32-10 normals; random-init weights of the workload's shape)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "F": w.F, "n_shared": w.S,
                   "gating": w.gating, "zipf_alpha": w.zipf_alpha, "path": path, "timing": timing},
        "tokens_per_s": tok_s,
        "active_tflop": {"experts": f_exp / 1e12, "router": f_rt / 1e12},
        "algorithmic_GBps": gbs,
        "hbm_frac": gbs / PEAK_HBM,
        "mfma_frac": tflops / peak_f,
        "path_ms": timed,
        "fused_speedup_vs_unfused": (timed["unfused"] / timed["fused"]) if len(timed) == 2 else None,
        "kernels": kernels,
        "experts_touched": touched,
        "max_group_rows": int(counts_np.max()),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
