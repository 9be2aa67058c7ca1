"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases span several tiles and ragged tails and are checked on every token;
the full-size workloads are checked on routing and dispatch for every token and
on outputs for a seeded sample of tokens (each token's output depends only on
its own row and the weights, so a sample is an exact sub-result).
"""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_layer_dispatch_amd as moe
import oracle
import synth
from synth import WORKLOADS, Workload
from moe_testlib import (FP8, TOL, cfg_of, check_dispatch, check_outputs, check_routing, check_rows, check_tokens_fp8,
                         check_xq, cover_rows, log, rel_l2, sample_tokens, to_dev, to_f64, upload)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_f32": WORKLOADS["tiny_f32"],
    "bf16_softmax_ragged": Workload("bf16_softmax_ragged", 2001, "bf16", 333, 256, 8, 2, 384, 0, "softmax"),
    "bf16_sigmoid_shared": Workload("bf16_sigmoid_shared", 2002, "bf16", 200, 384, 64, 6, 256, 1, "sigmoid",
                                    zipf_alpha=0.25),
    "bf16_sparse_groups": Workload("bf16_sparse_groups", 2003, "bf16", 37, 128, 96, 1, 128, 1, "softmax"),
    "bf16_k_equals_E": Workload("bf16_k_equals_E", 2004, "bf16", 70, 128, 8, 8, 128, 0, "softmax"),
    "f32_sigmoid_shared": Workload("f32_sigmoid_shared", 2005, "f32", 90, 256, 16, 3, 128, 1, "sigmoid",
                                   zipf_alpha=0.5),
    "fp8_softmax_shared": Workload("fp8_softmax_shared", 2006, "fp8_mxfp4", 150, 512, 32, 4, 256, 1, "softmax"),
    "fp8_sigmoid_zipf": Workload("fp8_sigmoid_zipf", 2007, "fp8_mxfp4", 300, 256, 64, 8, 384, 1, "sigmoid",
                                 zipf_alpha=0.25),
    "fp8_decode_1": Workload("fp8_decode_1", 2008, "fp8_mxfp4", 1, 512, 64, 8, 256, 1, "softmax"),
    "fp8_decode_5": Workload("fp8_decode_5", 2009, "fp8_mxfp4", 5, 512, 64, 8, 256, 1, "softmax"),
    "bf16_decode_3": Workload("bf16_decode_3", 2010, "bf16", 3, 256, 32, 4, 256, 1, "sigmoid"),
    # workgroup weight-streaming kernels (K slices of 1024): several rows per group, one to
    # four 128-column groups per workgroup tile
    "fp8_decode_wg_3": Workload("fp8_decode_wg_3", 2011, "fp8_mxfp4", 3, 2048, 64, 8, 1024, 1, "softmax"),
    "fp8_decode_wg_7": Workload("fp8_decode_wg_7", 2012, "fp8_mxfp4", 7, 2048, 64, 8, 1024, 1, "sigmoid",
                                zipf_alpha=0.25),
    # the router as a tiled GEMM (E a multiple of 256, T >= 2048) with a ragged last token tile
    "bf16_router_tiled": Workload("bf16_router_tiled", 2013, "bf16", 2100, 512, 256, 8, 128, 1, "sigmoid",
                                  zipf_alpha=0.25),
    # 256-row tiles with N a multiple of 256 (at least 160 rows per group): the 8-wave GEMM
    # tiles, and the persistent kernel's 512-thread variant -- bf16 with the one-pass
    # router, FP8 x FP4 with the tiled router
    "bf16_w8": Workload("bf16_w8", 2014, "bf16", 1024, 256, 8, 2, 256, 0, "softmax"),
    "fp8_w8_tiled_router": Workload("fp8_w8_tiled_router", 2015, "fp8_mxfp4", 5120, 256, 256, 8, 256, 1, "softmax"),
    # FP8 e4m3 x e4m3: 128-row tiles, ragged groups, 128- and 256-column tiles, decode sizes
    "fp8x8_softmax_shared": Workload("fp8x8_softmax_shared", 2016, "fp8_fp8", 150, 512, 32, 4, 256, 1, "softmax"),
    "fp8x8_sigmoid_zipf": Workload("fp8x8_sigmoid_zipf", 2017, "fp8_fp8", 300, 256, 64, 8, 384, 1, "sigmoid",
                                   zipf_alpha=0.25),
    "fp8x8_decode_3": Workload("fp8x8_decode_3", 2018, "fp8_fp8", 3, 384, 16, 4, 128, 1, "softmax"),
    "fp8x8_large_groups": Workload("fp8x8_large_groups", 2019, "fp8_fp8", 1200, 256, 8, 2, 256, 0, "softmax"),
    # weight streaming with 2048-wide K slices and tall row tiles: the shared expert's 20 rows
    # (more than 16 rows of 16 activation scales each), then up to 2.2 rows per group (row
    # tiles of 32 rows, several per group)
    "fp8_decode_tall_20": Workload("fp8_decode_tall_20", 2020, "fp8_mxfp4", 20, 1024, 256, 4, 2048, 1, "softmax"),
    # the persistent kernel's weight-stream phases at two workgroups per CU (few rows, small
    # staging buffers: four weight blocks in flight per wave), one and four column quads per
    # linear1 tile; tall_20 and rows_64 above take them at one workgroup per CU (eight blocks)
    "fp8_decode_stream_4": Workload("fp8_decode_stream_4", 2030, "fp8_mxfp4", 4, 1024, 64, 4, 2048, 1, "sigmoid"),
    "fp8_decode_stream_6": Workload("fp8_decode_stream_6", 2031, "fp8_mxfp4", 6, 1024, 256, 8, 2048, 1, "softmax"),
    "fp8_decode_rows_64": Workload("fp8_decode_rows_64", 2021, "fp8_mxfp4", 64, 1024, 256, 8, 2048, 1, "sigmoid",
                                   zipf_alpha=0.25),
    # no shared expert: G + 1 groups' plan words are an odd count (the staged rows behind them
    # start on the next 16 bytes)
    "fp8_decode_noshared": Workload("fp8_decode_noshared", 2022, "fp8_mxfp4", 7, 1024, 64, 4, 1024, 0, "softmax"),
}


def run_unfused(w, d, T=None):
    cfg = cfg_of(w, T)
    ws = moe.alloc_workspace(cfg)
    idx, gate, logits, keys = moe.route(cfg, d["x"], d["w_router"], d["bias"], ws=ws, want_logits=True)
    dsp = moe.dispatch(cfg, idx, d["x"], ws=ws)
    yp = moe.ffn(cfg, d["w1"], d["w2"], d["w1_scale"], d["w2_scale"], x=None if w.mode in FP8 else d["x"],
                 xq=dsp["xq"], xq_scale=dsp["xq_scale"], offsets=dsp["offsets"], row_to_slot=dsp["row_to_slot"],
                 ws=ws)
    y = moe.combine(cfg, yp, dsp["slot_to_row"], gate)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 0
    return cfg, ws, dict(idx=idx, gate=gate, logits=logits, keys=keys, dsp=dsp, y=y, y_perm=yp)


def run_fused(w, d, cfg, ws):
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")
    gate = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device="cuda")
    counts = torch.empty(cfg.G, dtype=torch.int32, device="cuda")
    y = moe.layer_fused(cfg, d["x"], d["w_router"], d["w1"], d["w2"], d["w1_scale"], d["w2_scale"], d["bias"],
                        ws=ws, topk_idx=idx, topk_gate=gate, counts=counts)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 0
    return y, idx, gate, counts


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_parity(name):
    w = SMALL[name]
    log(f"case {name}: mode={w.mode} T={w.T} d={w.d} E={w.E} k={w.k} F={w.F} S={w.S} {w.gating}")
    inp = synth.make_inputs(w)
    d = upload(inp)
    cfg, ws, r = run_unfused(w, d)
    near = check_routing(w, inp, r["idx"], r["gate"], r["logits"], r["keys"])
    check_dispatch(w, r["idx"], r["dsp"])
    if w.mode in FP8:
        check_xq(w, inp, r["dsp"]["xq"], r["dsp"]["xq_scale"])
    err = check_outputs(w, inp, r["y"], r["idx"], r["gate"], np.arange(w.T))
    # every expert output row, and in FP8 mode every row's h codes and scales
    check_rows(w, inp, r["dsp"], r["y_perm"], np.arange(w.T * (w.k + w.S)), ws=ws, cfg=cfg)
    if w.mode in FP8:
        check_tokens_fp8(w, inp, r["y"], r["dsp"], r["gate"], ws, cfg, np.arange(w.T))
    # the fused entry point gives the same bits
    y2, idx2, gate2, counts2 = run_fused(w, d, cfg, ws)
    assert torch.equal(idx2, r["idx"]) and torch.equal(gate2, r["gate"])
    assert torch.equal(counts2, r["dsp"]["counts"])
    assert torch.equal(y2.view(torch.int16 if w.mode != "f32" else torch.int32),
                       r["y"].view(torch.int16 if w.mode != "f32" else torch.int32)), "fused != unfused"
    # repeated calls give the same bits
    _, _, r2 = run_unfused(w, d)
    assert torch.equal(r2["y"], r["y"]) and torch.equal(r2["dsp"]["row_to_slot"], r["dsp"]["row_to_slot"])
    log(f"case {name}: rel L2 {err:.2e} (tol {TOL[w.mode]:.0e}), near-tie tokens {near}")


@pytest.mark.parametrize("name", ["bf16_sigmoid_shared", "f32_sigmoid_shared", "fp8_softmax_shared", "fp8_decode_5",
                                  "bf16_w8", "fp8_w8_tiled_router", "fp8x8_sigmoid_zipf", "fp8_decode_rows_64",
                                  "fp8_decode_tall_20", "fp8_decode_stream_6"])
def test_fused_grid_sizes_and_repeats(name):
    """The persistent kernel gives the unfused bits on a full grid, on 8 CUs and on 3 CUs
    (many items per workgroup), call after call (each launch leaves its counters clean for
    the next; a stale counter would let a step run early or time out)."""
    w = SMALL[name]
    log(f"case {name}: fused at several grid sizes")
    d = upload(synth.make_inputs(w))
    cfg, ws, r = run_unfused(w, d)
    view = torch.int16 if w.mode != "f32" else torch.int32
    for cu_limit in (0, 8, 3, 0):
        cfg_l = dataclasses.replace(cfg_of(w), cu_limit=cu_limit)
        y2, idx2, gate2, _ = run_fused(w, d, cfg_l, ws)
        assert torch.equal(idx2, r["idx"]) and torch.equal(gate2, r["gate"])
        assert torch.equal(y2.view(view), r["y"].view(view)), f"fused != unfused at cu_limit {cu_limit}"


def test_zero_tokens_is_noop():
    w = SMALL["bf16_softmax_ragged"]
    cfg = cfg_of(w, 0)
    x = torch.empty(0, w.d, dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros(w.E, w.d, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    idx, gate, _, _ = moe.route(cfg, x, wr, None, ws=ws)
    assert idx.numel() == 0


def test_all_tokens_same_experts_and_empty_groups():
    """A large bias on k experts sends every token there: k groups of T rows, the rest empty."""
    w = Workload("hot", 2011, "bf16", 130, 256, 16, 2, 128, 1, "softmax")
    inp = synth.make_inputs(w)
    inp["bias"] = np.zeros(w.E, np.float32)
    inp["bias"][[3, 11]] = 1000.0
    d = upload(inp)
    cfg, ws, r = run_unfused(w, d)
    counts = r["dsp"]["counts"].cpu().numpy()
    assert counts[3] == counts[11] == w.T and counts[w.E] == w.T and counts.sum() == w.T * (w.k + 1)
    check_routing(w, inp, r["idx"], r["gate"], r["logits"], r["keys"])
    check_dispatch(w, r["idx"], r["dsp"])
    check_outputs(w, inp, r["y"], r["idx"], r["gate"], np.arange(w.T))


def test_integer_grid_logits_exact():
    """Integer inputs make every fp32 partial sum exact: GPU logits equal the oracle's bit for bit."""
    for mode, E in (("bf16", 64), ("bf16", 8), ("f32", 8)):
        w = Workload("grid", 2012, mode, 100, 256, E, 2, 128, 0, "softmax")
        inp = synth.make_inputs(w, grid=True)
        d = upload(inp)
        cfg = cfg_of(w)
        ws = moe.alloc_workspace(cfg)
        _, _, logits, _ = moe.route(cfg, d["x"], d["w_router"], None, ws=ws, want_logits=True)
        np.testing.assert_array_equal(logits.cpu().numpy(), oracle.route(inp)["logits"])


def test_bad_indices_set_device_error():
    w = SMALL["bf16_sigmoid_shared"]
    cfg = cfg_of(w, 4)
    ws = moe.alloc_workspace(cfg)
    idx = torch.tensor([[0, 1, 2, 3, 4, 5]] * 4, dtype=torch.int32, device="cuda")
    idx[2, 3] = w.E  # out of range
    moe.dispatch(cfg, idx, None, ws=ws)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 1
    moe.clear_device_error(cfg, ws)
    assert moe.read_device_error(cfg, ws) == 0
    idx[2, 3] = 1  # duplicate of choice 1
    moe.dispatch(cfg, idx, None, ws=ws)
    assert moe.read_device_error(cfg, ws) == 2


def test_nonfinite_keys_set_device_error():
    w = SMALL["bf16_softmax_ragged"]
    inp = synth.make_inputs(w.with_T(8))
    d = upload(inp)
    d["x"][3, 5] = float("inf")
    cfg = cfg_of(w, 8)
    ws = moe.alloc_workspace(cfg)
    moe.route(cfg, d["x"], d["w_router"], None, ws=ws)
    assert moe.read_device_error(cfg, ws) == 3


def test_e4m3_quantiser_every_bf16_value():
    """Every finite bf16 value, in 128-blocks of similar magnitude, quantised bit-exactly."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = synth.bf16_to_f32(bits)
    keep = np.isfinite(vals)
    bits = bits[keep]
    order = np.argsort(np.abs(synth.bf16_to_f32(bits)), kind="stable")
    bits = bits[order]
    n = (bits.size // 1024) * 1024
    x = bits[:n].reshape(-1, 1024)
    T = x.shape[0]
    w = Workload("q", 1, "fp8_mxfp4", T, 1024, 8, 1, 128, 0, "softmax")
    cfg = cfg_of(w)
    ws = moe.alloc_workspace(cfg)
    idx = torch.zeros(T, 1, dtype=torch.int32, device="cuda")
    dsp = moe.dispatch(cfg, idx, to_dev(x, "bf16"), ws=ws)
    check_xq(w, {"x": x}, dsp["xq"], dsp["xq_scale"])


# ---- full-size workloads ----------------------------------------------------------

_CACHE = {}


def _full_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        w = WORKLOADS[name]
        if w.t_values:
            w = w.with_T(max(w.t_values))
        log(f"generating {name} inputs (T={w.T})")
        inp = synth.make_inputs(w)
        log("uploading")
        _CACHE[name] = (inp, upload(inp))
        log("inputs ready")
    return _CACHE[name]


FULL = [("mixtral_bf16", 4096), ("dsv3_bf16", 8192), ("dsv3_fp8fp4", 512), ("dsv3_fp8fp4", 8192),
        ("dsv3_fp8fp4", 32768), ("decode_fp8fp4", 1), ("decode_fp8fp4", 64), ("dsv3_fp8fp8", 8192)]


@pytest.mark.slow
@pytest.mark.parametrize("name,T", FULL, ids=[f"{n}-T{t}" for n, t in FULL])
def test_full_size_parity(name, T):
    inp_all, d_all = _full_inputs(name)
    w = inp_all["workload"].with_T(T)
    inp = dict(inp_all, workload=w, x=inp_all["x"][:T])
    d = dict(d_all, x=d_all["x"][:T])
    log(f"full {name} T={T}: running the HIP path")
    cfg, ws, r = run_unfused(w, d, T)
    log("routing and dispatch checks (all tokens)")
    near = check_routing(w, inp, r["idx"], r["gate"], r["logits"], r["keys"])
    check_dispatch(w, r["idx"], r["dsp"])
    toks = sample_tokens(T, 48, seed=T)
    if w.mode in FP8:
        check_xq(w, inp, r["dsp"]["xq"], r["dsp"]["xq_scale"], tokens=toks)
    log(f"oracle on {len(toks)} sampled tokens")
    err = check_outputs(w, inp, r["y"], r["idx"], r["gate"], toks)
    # one row in every 128-row block of every group: every (group, row tile) of the GEMMs
    # and both halves of any tile the tail split runs as two
    rows = cover_rows(r["dsp"]["offsets"].cpu().numpy(), 128 if T > 64 else 32, seed=T)
    log(f"oracle on {rows.size} rows covering every 128-row block of every group")
    agg, worst, mism = check_rows(w, inp, r["dsp"], r["y_perm"], rows, ws=ws, cfg=cfg)
    log(f"rows: rel L2 {agg:.2e}, worst row {worst:.2e}, h code mismatches {mism}")
    if w.mode in FP8:
        check_tokens_fp8(w, inp, r["y"], r["dsp"], r["gate"], ws, cfg, toks)
    y2, idx2, _, _ = run_fused(w, d, cfg, ws)
    assert torch.equal(idx2, r["idx"])
    assert torch.equal(y2.view(torch.int16), r["y"].view(torch.int16)), "fused != unfused"
    if w.mode == "fp8_mxfp4" and T <= 512:
        # the persistent kernel's weight-stream phases on few workgroups (a stream of many
        # tiles each), bitwise against the step chain again
        for cu_limit in (8, 3):
            log(f"full {name} T={T}: persistent kernel on {cu_limit} CUs")
            y3, _, _, _ = run_fused(w, d, dataclasses.replace(cfg, cu_limit=cu_limit), ws)
            assert torch.equal(y3.view(torch.int16), r["y"].view(torch.int16)), f"fused on {cu_limit} CUs != unfused"
    log(f"full {name} T={T}: rel L2 {err:.2e}, near-tie tokens {near}")
