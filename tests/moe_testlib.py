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

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8_mxfp4": 1e-2, "fp8_fp8": 1e-2}
FP8 = ("fp8_mxfp4", "fp8_fp8")  # modes with FP8 e4m3 activations (x and h quantised in-layer)


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
    wk = "u8" if w.mode in FP8 else act
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
    if w.mode not in FP8:
        # every token on its own as well (a token's output depends only on its row and the
        # weights); in FP8 mode a token's h codes may sit one step apart at a rounding midpoint,
        # which moves a single token by up to about 1e-2 at small F, so there the per-token check
        # takes the GPU's own h codes (check_tokens_fp8)
        assert_per_row(y_gpu, y_ref, tol, tokens, "token")
    return err


def assert_per_row(got, ref, tol, ids, what):
    per = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    nz = np.linalg.norm(ref, axis=1) > 0
    if not nz.any():
        return 0.0
    worst = int(np.argmax(np.where(nz, per, 0.0)))
    assert per[worst] <= tol, f"{what} {ids[worst]}: rel L2 {per[worst]:.3e} > {tol:.1e}"
    return float(per[worst])


# ---- per-row checks: the expert output (y_perm) and FP8 h of chosen dispatched rows -------

def row_tokens(w: Workload, r2s: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Token feeding each dispatched row: routed rows carry slot t*k + j, shared rows are T*k + t."""
    tk = w.T * w.k
    rows = np.asarray(rows, dtype=np.int64)
    return np.where(rows < tk, r2s[np.minimum(rows, tk - 1)] // w.k, rows - tk)


def row_groups(offsets: np.ndarray, rows: np.ndarray) -> np.ndarray:
    return np.searchsorted(offsets, np.asarray(rows, dtype=np.int64), side="right") - 1


def cover_rows(offsets: np.ndarray, block: int = 128, seed: int = 0) -> np.ndarray:
    """One seeded row in every block of `block` rows of every group (blocks start at the
    group's first row, as the GEMM row tiles and their 128-row halves do)."""
    rng = np.random.default_rng(seed)
    out = []
    for g in range(offsets.size - 1):
        a, b = int(offsets[g]), int(offsets[g + 1])
        for s in range(a, b, block):
            out.append(int(rng.integers(s, min(s + block, b))))
    return np.array(out, dtype=np.int64)


def oracle_rows(inp: dict, groups: np.ndarray, tokens: np.ndarray, want_h: bool = False, threads: int = 16):
    """Oracle expert outputs (and h before FP8 rounding) of the rows (group, token), computed
    by `threads` concurrent calls into the C oracle."""
    from concurrent.futures import ThreadPoolExecutor

    w = inp["workload"]
    n = len(groups)
    out = np.empty((n, w.d), dtype=np.float64)
    h = np.empty((n, w.F), dtype=np.float64) if want_h else None

    def job(i):
        xin = oracle.input_rows(inp, [int(tokens[i])])
        r = oracle.expert_rows(inp, int(groups[i]), xin, want_h=want_h)
        if want_h:
            out[i], h[i] = r[0][0], r[1][0]
        else:
            out[i] = r[0]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(job, range(n)))
    return out, h


def check_rows(w: Workload, inp: dict, dsp: dict, y_perm, rows: np.ndarray, ws=None, cfg=None, tol=None):
    """The GPU's expert output rows (y_perm) against the oracle, row by row (rel L2 each, and
    over all of them); in FP8 mode also the GPU's h codes and scales of those rows against
    the oracle's rule applied to the oracle's h (fp32): scales equal wherever the block
    maximum is clear of a power-of-two boundary, and codes equal except single steps at a
    rounding midpoint.  Returns (aggregate rel L2, worst row rel L2, code mismatches)."""
    import e4m3_ref

    tol = TOL[w.mode] if tol is None else tol
    offs = dsp["offsets"].cpu().numpy()
    r2s = dsp["row_to_slot"].cpu().numpy()
    groups = row_groups(offs, rows)
    toks = row_tokens(w, r2s, rows)
    fp8 = w.mode in FP8
    ref, h = oracle_rows(inp, groups, toks, want_h=fp8)
    got = to_f64(y_perm[torch.from_numpy(rows).to(y_perm.device)])
    assert np.all(np.isfinite(got)), "non-finite expert output"
    if fp8:
        # linear2 of the GPU's own h codes (the oracle dequantising the identical codes)
        ref = down_of_gpu_h(w, inp, ws, cfg, rows, groups)
    worst = assert_per_row(got, ref, tol, rows, "row")
    agg = rel_l2(got, ref)
    assert agg <= tol
    mism = 0
    if fp8:
        nrows = w.T * (w.k + w.S)
        codes_all = moe.workspace_region(cfg, ws, "h").view(nrows, w.F)
        scales_all = moe.workspace_region(cfg, ws, "h_scale").view(torch.float32).view(nrows, w.F // 128)
        idx = torch.from_numpy(rows).to(codes_all.device)
        g_codes = codes_all[idx].cpu().numpy()
        g_scales = scales_all[idx].cpu().numpy()
        hf = h.astype(np.float32)
        o_codes, o_scales = oracle.quant_e4m3_b128(hf)
        amax = np.abs(hf).reshape(len(rows), -1, 128).max(axis=2).astype(np.float64)
        # a block whose maximum lies within 1e-4 of a power-of-two scale boundary may take
        # either exponent when h is computed in another summation order
        lo = np.array([[oracle.e4m3_block_exponent(float(a * (1 - 1e-4))) for a in r] for r in amax])
        hi = np.array([[oracle.e4m3_block_exponent(float(a * (1 + 1e-4))) for a in r] for r in amax])
        clear = lo == hi
        assert np.array_equal(g_scales[clear], o_scales[clear]), "h block scales differ"
        same_scale = (g_scales == o_scales)
        cmp = np.repeat(same_scale, 128, axis=1)
        diff = (g_codes != o_codes) & cmp
        mism = int(diff.sum())
        if mism:
            gi, gj = np.nonzero(diff)
            gc, oc = g_codes[gi, gj], o_codes[gi, gj]
            v = hf[gi, gj].astype(np.float64) / o_scales[gi, gj // 128]  # the oracle's h, scaled
            # The GPU's h is an fp32 sum in another order (and, on the MFMA, another internal
            # rounding): its error scales with the block's terms rather than with the element, so
            # it is bounded relative to the block maximum (448 in scaled units), at 1e-4 of it.
            # The GPU's code must be a round-to-nearest-even of some value within that distance
            # of the oracle's h: between the codes of v - delta and v + delta.
            delta = 448.0 * 1e-4
            lo = e4m3_ref.decode_codes(e4m3_ref.encode_bits((v - delta).astype(np.float32).view(np.uint32)))
            hi = e4m3_ref.decode_codes(e4m3_ref.encode_bits((v + delta).astype(np.float32).view(np.uint32)))
            gv = e4m3_ref.decode_codes(gc)
            ok = (gv >= lo) & (gv <= hi)
            bad = np.nonzero(~ok)[0][:5]
            assert ok.all(), ("h code is no rounding of a value near the oracle's h: " +
                              "; ".join(f"row {rows[gi[b]]} col {gj[b]}: scaled oracle h {v[b]:.6g}, gpu code "
                                        f"{gv[b]:.6g}, oracle code {e4m3_ref.decode_codes(oc[b:b + 1])[0]:.6g}"
                                        for b in bad))
            assert mism <= 1e-2 * cmp.sum(), f"{mism} of {int(cmp.sum())} h codes differ"
    return agg, worst, mism


def gpu_hhat(w: Workload, ws, cfg, rows: np.ndarray) -> np.ndarray:
    """The GPU's FP8 h of dispatched rows, dequantised with the oracle's e4m3 decoder: code x scale."""
    import e4m3_ref

    nrows = w.T * (w.k + w.S)
    codes = moe.workspace_region(cfg, ws, "h").view(nrows, w.F)
    scales = moe.workspace_region(cfg, ws, "h_scale").view(torch.float32).view(nrows, w.F // 128)
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(codes.device)
    c = codes[idx].cpu().numpy()
    sc = scales[idx].cpu().numpy().astype(np.float64)
    return e4m3_ref.decode_codes(c) * np.repeat(sc, 128, axis=1)


def down_of_gpu_h(w: Workload, inp: dict, ws, cfg, rows: np.ndarray, groups: np.ndarray, threads: int = 16):
    from concurrent.futures import ThreadPoolExecutor

    hh = gpu_hhat(w, ws, cfg, rows)
    out = np.empty((len(rows), w.d), dtype=np.float64)

    def job(i):
        out[i] = oracle.down_rows(inp, int(groups[i]), hh[i:i + 1])[0]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(job, range(len(rows))))
    return out


def check_tokens_fp8(w: Workload, inp: dict, y, dsp: dict, gate, ws, cfg, tokens, tol=None):
    """FP8 mode, token by token: the GPU's y against the gate-weighted sum, in the layer's
    fixed order, of the oracle's linear2 of the GPU's own h codes of the token's rows."""
    tol = TOL[w.mode] if tol is None else tol
    tokens = np.asarray(tokens, dtype=np.int64)
    s2r = dsp["slot_to_row"].cpu().numpy()
    offs = dsp["offsets"].cpu().numpy()
    g_np = gate.cpu().numpy().astype(np.float64)
    rows = [s2r[t * w.k + j] for t in tokens for j in range(w.k)]
    if w.S:
        rows += [w.T * w.k + t for t in tokens]
    rows = np.array(rows, dtype=np.int64)
    o = down_of_gpu_h(w, inp, ws, cfg, rows, row_groups(offs, rows))
    n = len(tokens)
    ref = np.zeros((n, w.d))
    for i in range(n):
        for j in range(w.k):
            ref[i] += g_np[tokens[i], j] * o[i * w.k + j]
        if w.S:
            ref[i] += o[n * w.k + i]
    got = to_f64(y)[tokens]
    return assert_per_row(got, ref, tol, tokens, "token")
