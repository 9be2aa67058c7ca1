"""The dense FP8 x MXFP4 GEMM and one expert-parallel rank's expert FFNs over its receive
buffer, on the GPU through the C ABI, against the oracle.

Operands are seeded synthetic FP8 rows (e4m3 codes with power-of-two block scales) and
MXFP4 weights from the generators, so both sides start from identical codes."""
import math

import numpy as np
import pytest
import torch

import mixture_experts_layer_dispatch_amd as moe
import oracle
import synth
from synth import Workload
from moe_testlib import TOL, log, rel_l2, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _gemm_case(M, N, K, seed, grid=False):
    if grid:
        a, a_s = synth.fp8_rows(seed, 1, M, K, 0.0, grid=(-3, 3))
        b, b_s = synth.mxfp4(seed, 2, 1, N, K, 0.0, grid=(-2, 2))
    else:
        a, a_s = synth.fp8_rows(seed, 1, M, K, 1.0)
        b, b_s = synth.mxfp4(seed, 2, 1, N, K, 1.0 / math.sqrt(K))
    return a, a_s, b[0], b_s[0]


def _run_gemm(a, a_s, b, b_s):
    c = moe.gemm_fp8_mxfp4(to_dev(a, "u8"), to_dev(a_s, "f32"), to_dev(b, "u8"), to_dev(b_s, "u8"))
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("M,N,K", [(300, 384, 512), (5, 128, 128), (1000, 512, 1024), (700, 768, 256)])
def test_dense_gemm_matches_oracle(M, N, K):
    log(f"dense FP8 x MXFP4 GEMM M={M} N={N} K={K}")
    a, a_s, b, b_s = _gemm_case(M, N, K, 6000 + M)
    c = to_f64(_run_gemm(a, a_s, b, b_s))
    ref = oracle.gemm_fp8_mxfp4(a, a_s, b, b_s)
    per = np.linalg.norm(c - ref, axis=1) / np.linalg.norm(ref, axis=1)
    # identical codes on both sides: fp32 sums and the bf16 output rounding (2^-9) remain
    assert per.max() <= 1e-2 and rel_l2(c, ref) <= 5e-3, f"worst row {per.max():.3e}"


def test_dense_gemm_integer_grid_is_exact():
    """Integer operands: every fp32 partial sum is exact, so C equals the oracle rounded to bf16."""
    for M, N, K in ((300, 256, 256), (64, 384, 128)):
        a, a_s, b, b_s = _gemm_case(M, N, K, 6100 + M, grid=True)
        c = _run_gemm(a, a_s, b, b_s).view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle.gemm_fp8_mxfp4(a, a_s, b, b_s)
        np.testing.assert_array_equal(c, synth.f32_to_bf16(ref.astype(np.float32)))


# ---- one expert-parallel rank --------------------------------------------------------------

def _ep_case(E, n_src, T, d, F, seed, counts=None, slack=0, mean=20):
    w = Workload("ep", seed, "fp8_mxfp4", T, d, E, 1, F, 1, "softmax")
    rng = np.random.default_rng(seed)
    if counts is None:
        counts = rng.poisson(mean, size=(E, n_src)).astype(np.int32)
        counts[0, 0] = 0
        counts[E - 1, :] = 0  # an expert nothing was sent to
    R = int(counts.sum())
    cap = R + slack
    w1, w1s = synth.mxfp4(seed, synth.TID_W1, E + 1, 2 * F, d, 1.0 / math.sqrt(d))
    w2, w2s = synth.mxfp4(seed, synth.TID_W2, E + 1, d, F, 1.0 / math.sqrt(F))
    rq, rs = synth.fp8_rows(seed, 11, max(cap, 1), d, 1.0)
    xq, xs = synth.fp8_rows(seed, 12, T, d, 1.0)
    inp = {"workload": w, "w1": w1, "w1_scale": w1s, "w2": w2, "w2_scale": w2s}
    return w, inp, counts, cap, (rq[:cap], rs[:cap]), (xq, xs)


def _run_ep(w, inp, counts, cap, recv, own):
    cfg = moe.Config(T=w.T, d=w.d, E=w.E, k=1, F=w.F, n_shared=1, mode="fp8_mxfp4")
    ws = moe.ep_workspace(cfg, cap)
    yr, ysh = moe.ep_ffn(cfg, to_dev(inp["w1"], "u8"), to_dev(inp["w2"], "u8"), to_dev(inp["w1_scale"], "u8"),
                         to_dev(inp["w2_scale"], "u8"), recv_counts=to_dev(counts, "i32"),
                         recv_xq=to_dev(recv[0], "u8"), recv_xs=to_dev(recv[1], "f32"), xq=to_dev(own[0], "u8"),
                         xs=to_dev(own[1], "f32"), ws=ws)
    torch.cuda.synchronize()
    return cfg, ws, yr, ysh


def _oracle_rows(inp, groups, codes, scales, threads=16):
    """Oracle expert outputs of given FP8 rows (concurrent calls into the C oracle)."""
    from concurrent.futures import ThreadPoolExecutor

    w = inp["workload"]
    out = np.empty((len(groups), w.d), dtype=np.float64)

    def job(i):
        xin = oracle.dequant_e4m3_rows(codes[i:i + 1], scales[i:i + 1])
        out[i] = oracle.expert_rows(inp, int(groups[i]), xin)[0]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(job, range(len(groups))))
    return out


def _check_ep_rows(w, inp, counts, recv, own, yr, ysh, rows, own_rows, per_row_tol):
    offs = np.concatenate([[0], np.cumsum(counts.sum(axis=1))])
    groups = np.searchsorted(offs, rows, side="right") - 1
    codes = np.concatenate([recv[0][rows], own[0][own_rows]])
    scales = np.concatenate([recv[1][rows], own[1][own_rows]])
    ref = _oracle_rows(inp, np.concatenate([groups, np.full(len(own_rows), w.E)]), codes, scales)
    got = np.concatenate([to_f64(yr[torch.from_numpy(rows).cuda()]), to_f64(ysh[torch.from_numpy(own_rows).cuda()])])
    per = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    err = rel_l2(got, ref)
    assert np.all(np.isfinite(got))
    # FP8 tolerance over all rows; a row alone may move further where an h code sits one step
    # away at a rounding midpoint (about 0.06 |h_f| / ||h|| of the row)
    assert err <= TOL["fp8_mxfp4"] and per.max() <= per_row_tol, f"rel L2 {err:.3e}, worst row {per.max():.3e}"
    return err, float(per.max())


def test_ep_ffn_small():
    w, inp, counts, cap, recv, own = _ep_case(4, 3, 50, 256, 256, 6200, slack=9)
    log(f"EP shard: E_local={w.E}, sources {counts.shape[1]}, {int(counts.sum())} received rows, T={w.T}")
    cfg, ws, yr, ysh = _run_ep(w, inp, counts, cap, recv, own)
    assert moe.read_device_error(cfg, ws) == 0
    R = int(counts.sum())
    err, worst = _check_ep_rows(w, inp, counts, recv, own, yr, ysh, np.arange(R), np.arange(w.T), 3e-2)
    log(f"EP shard: rel L2 {err:.2e}, worst row {worst:.2e}")


def test_ep_ffn_overflow_is_reported_and_bounded():
    """More rows announced than the buffer holds: the device error word says so, and the rows
    that fit are still computed (nothing reaches past the buffer)."""
    w, inp, counts, cap, recv, own = _ep_case(3, 2, 20, 128, 128, 6201)
    counts_big = counts.copy()
    counts_big[1, 1] += 40
    cfg, ws, yr, ysh = _run_ep(w, inp, counts_big, cap, recv, own)
    assert moe.read_device_error(cfg, ws) == 5
    R0 = int(counts[0].sum())
    _check_ep_rows(w, inp, counts_big, recv, own, yr, ysh, np.arange(R0), np.arange(4), 3e-2)


@pytest.mark.slow
def test_ep_ffn_full_rank_shape():
    """The DeepSeek-V3 FP8 x FP4 shape at EP8: 32 local experts plus the shared one, the rows
    8 ranks x 8192 tokens send to them under uniform top-8 routing (about 65,536), and the
    rank's own 8192 tokens; one row of every 128-row block of every expert is checked."""
    E, n_src, T, d, F = 32, 8, 8192, 7168, 2048
    rng = np.random.default_rng(6300)
    counts = np.zeros((E, n_src), dtype=np.int32)
    for s in range(n_src):
        choice = np.argsort(rng.random((T, 256)), axis=1)[:, :8]  # uniform 8-of-256 per token
        c = np.bincount(choice.reshape(-1), minlength=256)[:E]
        counts[:, s] = c
    w, inp, counts, cap, recv, own = _ep_case(E, n_src, T, d, F, 6300, counts=counts)
    log(f"EP shard full: {int(counts.sum())} received rows")
    cfg, ws, yr, ysh = _run_ep(w, inp, counts, cap, recv, own)
    assert moe.read_device_error(cfg, ws) == 0
    offs = np.concatenate([[0], np.cumsum(counts.sum(axis=1))])
    rows = np.array([int(rng.integers(s, min(s + 128, offs[g + 1]))) for g in range(E)
                     for s in range(offs[g], offs[g + 1], 128)], dtype=np.int64)
    own_rows = np.arange(0, T, 128) + rng.integers(0, 128, size=T // 128)
    err, worst = _check_ep_rows(w, inp, counts, recv, own, yr, ysh, rows, own_rows, 1e-2)
    log(f"EP shard full: rel L2 {err:.2e}, worst row {worst:.2e} over {rows.size + own_rows.size} rows")
