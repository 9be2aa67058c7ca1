"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, and compare it with the CPU oracle."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import mixture_experts_layer_dispatch_amd as moe
import oracle
import synth
from synth import Workload

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8_mxfp4": 1e-2}


def log(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def cfg_of(w: Workload, T: int | None = None) -> moe.Config:
    return moe.Config(T=w.T if T is None else T, d=w.d, E=w.E, k=w.k, F=w.F, n_shared=w.S, gating=w.gating,
                      mode=w.mode)


def to_dev(a, kind: str, device="cuda"):
    if a is None:
        return None
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(inp: dict) -> dict:
    w = inp["workload"]
    act = "f32" if w.mode == "f32" else "bf16"
    wk = "u8" if w.mode == "fp8_mxfp4" else act
    return {
        "x": to_dev(inp["x"], act),
        "w_router": to_dev(inp["w_router"], act),
        "bias": to_dev(inp["bias"], "f32"),
        "w1": to_dev(inp["w1"], wk),
        "w2": to_dev(inp["w2"], wk),
        "w1_scale": to_dev(inp["w1_scale"], "u8"),
        "w2_scale": to_dev(inp["w2_scale"], "u8"),
    }


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid])).astype(np.int64)


def check_routing(w: Workload, inp: dict, idx, gate, logits, keys, margin_tol: float = 1e-4):
    """Routing contract.

    (i)  bit-exact: the oracle's top-k over the GPU's keys equals the GPU's indices;
    (ii) GPU logits against the oracle's (rel L2 <= 1e-5); GPU keys against the oracle's
         keys recomputed from the GPU logits (<= 2 ulp); gates within 1e-5 relative;
    (iii) on every token whose oracle margin between the k-th and (k+1)-th key exceeds
         margin_tol * max(1, |key|), the GPU selects the oracle's set of experts, in an order
         the oracle's own keys agree with up to that tolerance (near-equal keys inside the
         top-k may swap places when the two sides compute logits independently).
    Returns the number of near-tie tokens excluded from (iii).
    """
    T = idx.shape[0]
    idx_n, gate_n = idx.cpu().numpy(), gate.cpu().numpy()
    lg_n, ky_n = logits.cpu().numpy(), keys.cpu().numpy()
    o_idx, o_gate = oracle.topk_gates_from(w, lg_n, ky_n)
    np.testing.assert_array_equal(idx_n, o_idx, err_msg="top-k over the GPU keys differs")
    np.testing.assert_allclose(gate_n, o_gate, rtol=1e-5, atol=1e-6, err_msg="gates")
    bias = inp["bias"]
    o_keys = oracle.keys_from_logits(w, lg_n, bias)
    ulp = np.abs(ky_n.view(np.int32).astype(np.int64) - o_keys.view(np.int32).astype(np.int64))
    same_sign = np.sign(ky_n) == np.sign(o_keys)
    assert np.all(ulp[same_sign] <= 2) and np.allclose(ky_n[~same_sign], o_keys[~same_sign], atol=1e-6), \
        f"keys differ by up to {ulp[same_sign].max()} ulp"
    ref = oracle.route(inp, T=T)
    assert rel_l2(lg_n.astype(np.float64), ref["logits"].astype(np.float64)) <= 1e-5, "logits rel L2"
    srt = -np.sort(-ref["keys"], axis=1)
    if w.k < w.E:
        margin = srt[:, w.k - 1] - srt[:, w.k]
        thr = margin_tol * np.maximum(1.0, np.abs(srt[:, w.k - 1]))
        clear = margin > thr
    else:
        clear = np.ones(T, bool)
    same_set = np.all(np.sort(ref["idx"], 1) == np.sort(idx_n, 1), axis=1)
    bad = np.where(clear & ~same_set)[0]
    assert bad.size == 0, f"selected experts differ from the oracle's on clear-margin tokens {bad[:10]}"
    k_gpu = np.take_along_axis(ref["keys"], idx_n.astype(np.int64), 1)   # oracle keys in GPU order
    tol = margin_tol * np.maximum(1.0, np.abs(k_gpu[:, :-1]))
    order_ok = np.all(k_gpu[:, :-1] >= k_gpu[:, 1:] - tol, axis=1)
    bad = np.where(clear & ~order_ok)[0]
    assert bad.size == 0, f"GPU order contradicts the oracle's keys on tokens {bad[:10]}"
    return int((~clear).sum())


def check_dispatch(w: Workload, idx, dsp):
    """Bit-exact counts, offsets and both permutations against the oracle fed the GPU's indices."""
    ref = oracle.dispatch(w, idx.cpu().numpy())
    for key in ("counts", "offsets", "slot_to_row", "row_to_slot"):
        np.testing.assert_array_equal(dsp[key].cpu().numpy(), ref[key], err_msg=key)
    return ref


def check_xq(w: Workload, inp: dict, xq, xs, tokens=None):
    """FP8 activation codes and scales bit-exact against the oracle's quantiser."""
    x = inp["x"] if tokens is None else inp["x"][tokens]
    codes, scales = oracle.quant_e4m3_b128(synth.bf16_to_f32(x))
    g_codes = xq.cpu().numpy() if tokens is None else xq.cpu().numpy()[tokens]
    g_scales = xs.cpu().numpy() if tokens is None else xs.cpu().numpy()[tokens]
    np.testing.assert_array_equal(g_codes, codes, err_msg="e4m3 codes")
    np.testing.assert_array_equal(g_scales, scales, err_msg="e4m3 scales")


def check_outputs(w: Workload, inp: dict, y, idx, gate, tokens, tol=None, nthreads=0):
    """rel L2 of the GPU output against the oracle fed the GPU's routing, on `tokens`."""
    tol = TOL[w.mode] if tol is None else tol
    y_ref, _, _ = oracle.layer(inp, tokens=tokens, idx=idx.cpu().numpy(), gates=gate.cpu().numpy(),
                               nthreads=nthreads)
    y_gpu = to_f64(y)[tokens]
    err = rel_l2(y_gpu, y_ref)
    assert np.all(np.isfinite(y_gpu)), "non-finite GPU output"
    assert err <= tol, f"output rel L2 {err:.3e} > {tol:.1e}"
    return err
