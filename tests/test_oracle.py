"""Pins for the CPU oracle and the input generator (CPU only).

Each test checks the oracle against something other than itself: a published
known-answer vector, an independent library routine (torch's float8 casts,
numpy's stable lexsort, scipy's softmax, torch fp64 matmuls), brute force on
tiny inputs, closed forms and invariants of the definitions.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from synth import Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- generator

def test_philox_known_answers():
    # Known-answer vectors published with the Random123 library (Salmon et al., SC'11).
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for case in kat["cases"]:
        got = synth.philox4x32_10([int(v, 16) for v in case["ctr"]], [int(v, 16) for v in case["key"]])
        assert [f"{v:08x}" for v in got] == case["out"]


def test_generator_subrange_and_threads_independent():
    whole = synth.normal(7, 3, (4099,), 0.5)
    part = synth.normal(7, 3, (1000,), 0.5, offset=1234)
    np.testing.assert_array_equal(whole[1234:2234], part)
    b = synth.normal(7, 3, (4099,), 0.5, dtype="bf16")
    np.testing.assert_array_equal(b, synth.f32_to_bf16(whole))
    assert abs(whole.mean()) < 0.05 and abs(whole.std() - 0.5) < 0.03


def test_generator_normal_moments():
    z = synth.normal(11, 1, (1 << 20,), 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3
    assert abs(z.var() - 1.0) < 5e-3
    assert abs((z ** 4).mean() - 3.0) < 0.05  # Gaussian kurtosis


def test_mxfp4_generator_reconstructs_within_half_step():
    codes, scales = synth.mxfp4(5, 4, 2, 8, 64, 0.1)
    vals = synth.normal(5, 4, (2 * 8 * 64,), 0.1).reshape(2, 8, 64)
    lut = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(2, 8, 64)
    deq = lut[nib] * np.exp2(np.repeat(scales.astype(np.int64) - 127, 32, axis=-1))
    blocks = vals.reshape(-1, 32)
    amax = np.abs(blocks).max(1)
    e = np.floor(np.log2(amax)) - 2
    np.testing.assert_array_equal(scales.reshape(-1), (e + 127).astype(np.uint8))
    # |v| / 2^e lies in [0, 8): half a grid step below 6 (at most 1 * 2^e), and
    # saturation to 6 above it (at most 2 * 2^e)
    err = np.abs(deq.reshape(-1, 32) - blocks)
    scaled = np.abs(blocks) / np.exp2(e)[:, None]
    assert np.all(err[scaled <= 6] <= np.exp2(np.broadcast_to(e[:, None], err.shape))[scaled <= 6] + 1e-12)
    assert np.all(err <= 2 * np.exp2(e)[:, None] + 1e-12)


# ---------------------------------------------------------------- formats

def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_e4m3_encode_matches_torch_rne():
    # every code value, every midpoint between neighbours (ties), and random values
    vals = sorted({oracle.e4m3_decode(c) for c in range(0x7F)})
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    rnd = np.random.default_rng(0).uniform(-448, 448, 20000).tolist()
    tiny = np.random.default_rng(1).uniform(-0.02, 0.02, 5000).tolist()
    probe = np.array(vals + mids + [-v for v in vals + mids] + rnd + tiny + [0.0, -0.0], dtype=np.float32)
    ref = torch.from_numpy(probe).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in probe], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)
    # saturation beyond the largest finite value (torch gives NaN there, the format rule saturates)
    assert oracle.e4m3_encode(1e6) == 0x7E and oracle.e4m3_encode(-500.0) == 0xFE


def test_e2m1_and_e8m0_tables():
    # OCP Microscaling Formats v1.0, the FP4 E2M1 value table.
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = oracle.e2m1_decode(c)
        assert v == (-1 if c & 8 else 1) * table[c & 7]
    assert oracle.e8m0_decode(127) == 1.0
    assert oracle.e8m0_decode(0) == 2.0 ** -127
    assert oracle.e8m0_decode(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0_decode(255))


def test_block_exponent_is_smallest_fitting_power():
    rng = np.random.default_rng(2)
    cands = list(rng.uniform(1e-6, 1e4, 2000).astype(np.float32))
    cands += [np.float32(448.0 * 2.0 ** p) for p in range(-20, 20)]
    cands += [np.nextafter(np.float32(448.0 * 2.0 ** p), np.float32(np.inf)) for p in range(-20, 20)]
    for a in cands:
        e = oracle.e4m3_block_exponent(float(a))
        assert float(a) <= 448.0 * 2.0 ** e
        assert float(a) > 448.0 * 2.0 ** (e - 1)
    assert oracle.e4m3_block_exponent(0.0) == 0


def test_quant_b128_roundtrip_and_bounds():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((4, 256)) * rng.uniform(0.01, 100, (4, 1))).astype(np.float32)
    codes, scales = oracle.quant_e4m3_b128(v)
    assert codes.shape == v.shape and scales.shape == (4, 2)
    # scales are powers of two and the block max lands in (224, 448]
    m, _ = np.frexp(scales)
    assert np.all(m == 0.5)
    blocks = v.reshape(4, 2, 128)
    amax = np.abs(blocks).max(-1)
    assert np.all(amax / scales <= 448) and np.all(amax / scales > 224)
    # codes agree with torch's RNE cast of v / scale (exact: division by a power of two)
    ref = torch.from_numpy((blocks / scales[..., None]).reshape(4, 256).astype(np.float32))
    ref = ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
    # dequantising the codes and quantising again returns the same codes
    deq = np.vectorize(oracle.e4m3_decode)(codes).reshape(4, 2, 128) * scales[..., None]
    c2, s2 = oracle.quant_e4m3_b128(deq.reshape(4, 256).astype(np.float32))
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)


# ---------------------------------------------------------------- routing

def _tiny(E, k, T=16, gating="softmax", d=4, S=0, F=128, mode="f32", alpha=0.0, seed=77):
    return Workload("t", seed, mode, T, d, E, k, F, S, gating, zipf_alpha=alpha)


def _route_inputs(w, logits, bias=None):
    """Inputs whose logits are exactly the given integers: x = one-hot rows, W_r = logits^T."""
    T, E = logits.shape
    x = np.eye(T, w.d, dtype=np.float32) if w.d >= T else None
    assert x is not None
    wr = np.zeros((E, w.d), dtype=np.float32)
    wr[:, :T] = logits.T
    return {"workload": w, "x": x, "w_router": wr, "bias": bias}


def _brute_topk(keys, k):
    E = len(keys)
    for S in itertools.combinations(range(E), k):
        Sset = set(S)
        ok = all(keys[i] > keys[j] or (keys[i] == keys[j] and i < j)
                 for i in S for j in range(E) if j not in Sset)
        if ok:
            return sorted(S, key=lambda i: (-keys[i], i))
    raise AssertionError("no valid subset")


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (8, 2), (7, 7)])
def test_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    T = 24
    logits = rng.integers(-2, 3, (T, E)).astype(np.float32)  # integer grid: many ties
    w = _tiny(E, k, T=T, d=T)
    r = oracle.route(_route_inputs(w, logits))
    for t in range(T):
        assert list(r["idx"][t]) == _brute_topk(list(logits[t]), k)
        # numpy's stable lexsort (descending key, ascending index) agrees
        assert list(r["idx"][t]) == list(np.lexsort((np.arange(E), -logits[t]))[:k])
    np.testing.assert_array_equal(r["logits"], logits)


def test_topk_all_equal_keys_picks_lowest_indices():
    w = _tiny(8, 3, T=4, d=4)
    r = oracle.route(_route_inputs(w, np.zeros((4, 8), np.float32)))
    assert np.all(r["idx"] == np.array([0, 1, 2]))
    np.testing.assert_allclose(r["gates"], 1.0 / 3.0, rtol=1e-7)


def test_softmax_gates_properties():
    rng = np.random.default_rng(5)
    T, E = 32, 8
    logits = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    for k in (1, 2, 5, 8):
        w = _tiny(E, k, T=T, d=T)
        r = oracle.route(_route_inputs(w, logits))
        np.testing.assert_allclose(r["gates"].sum(1), 1.0, rtol=1e-6)
        if k == 1:
            assert np.all(r["gates"] == 1.0)
        if k == E:
            # the full softmax (scipy) in descending order
            ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
            np.testing.assert_allclose(r["gates"], np.take_along_axis(ref, r["idx"], 1), rtol=1e-6)
        # softmax over all E, keep top-k, renormalise: the same gates
        full = scipy.special.softmax(logits.astype(np.float64), axis=1)
        sel = np.take_along_axis(full, r["idx"], 1)
        np.testing.assert_allclose(r["gates"], sel / sel.sum(1, keepdims=True), rtol=1e-6)
    # invariant to a constant added to every logit (exact shift by a power of two)
    w = _tiny(E, 3, T=T, d=T)
    r0 = oracle.route(_route_inputs(w, logits))
    r1 = oracle.route(_route_inputs(w, logits + np.float32(4.0)))
    np.testing.assert_array_equal(r0["idx"], r1["idx"])
    np.testing.assert_allclose(r0["gates"], r1["gates"], rtol=1e-6)


def test_bias_moves_selection_not_gates():
    rng = np.random.default_rng(6)
    T, E, k = 32, 8, 2
    logits = rng.standard_normal((T, E)).astype(np.float32)
    for gating in ("softmax", "sigmoid"):
        w = _tiny(E, k, T=T, d=T, gating=gating)
        r0 = oracle.route(_route_inputs(w, logits))
        # a large bias on expert 7 forces it into every token's selection
        bias = np.zeros(E, np.float32)
        bias[7] = 100.0
        r1 = oracle.route(_route_inputs(w, logits, bias))
        assert np.all((r1["idx"] == 7).any(1))
        # gates depend only on the chosen raw scores: recompute them from r1's selection
        for t in range(T):
            raw = logits[t, r1["idx"][t]].astype(np.float64)
            g = scipy.special.softmax(raw) if gating == "softmax" else scipy.special.expit(raw) / scipy.special.expit(raw).sum()
            np.testing.assert_allclose(r1["gates"][t], g, rtol=1e-6)
        # a bias that leaves the selection unchanged leaves the gates bit-identical
        small = np.full(E, 1e-3, np.float32)
        r2 = oracle.route(_route_inputs(w, logits, small))
        same = np.all(r2["idx"] == r0["idx"], 1)
        assert same.sum() > T // 2
        np.testing.assert_array_equal(r2["gates"][same], r0["gates"][same])


def test_sigmoid_keys_and_gates():
    rng = np.random.default_rng(8)
    T, E, k = 16, 16, 4
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = rng.uniform(0, 0.3, E).astype(np.float32)
    w = _tiny(E, k, T=T, d=T, gating="sigmoid")
    r = oracle.route(_route_inputs(w, logits, bias))
    s = scipy.special.expit(logits.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(r["keys"], s + bias)
    np.testing.assert_allclose(r["gates"].sum(1), 1.0, rtol=1e-6)


def test_route_rejects_nonfinite_keys():
    w = _tiny(4, 2, T=4, d=4)
    logits = np.zeros((4, 4), np.float32)
    logits[1, 2] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.route(_route_inputs(w, logits))


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,k,S", [(1, 4, 2, 0), (64, 8, 2, 0), (50, 16, 4, 1), (37, 256, 8, 1)])
def test_dispatch_invariants_and_brute_force(T, E, k, S):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = _tiny(E, k, T=T, S=S)
    d = oracle.dispatch(w, idx)
    counts, offs, s2r, r2s = d["counts"], d["offsets"], d["slot_to_row"], d["row_to_slot"]
    assert counts.sum() == T * k + S * T
    assert np.all(np.diff(offs) == counts) and offs[0] == 0 and offs[-1] == T * k + S * T
    np.testing.assert_array_equal(np.bincount(idx.ravel(), minlength=E), counts[:E])
    # bijection and inverse
    assert sorted(s2r.tolist()) == list(range(T * k))
    np.testing.assert_array_equal(r2s[s2r], np.arange(T * k))
    # brute force: slots stably sorted by expert (Python's sorted is stable)
    order = sorted(range(T * k), key=lambda s: idx.ravel()[s])
    np.testing.assert_array_equal(r2s, np.array(order, dtype=np.int32))
    # within each expert, ascending token order
    for e in range(E):
        rows = r2s[offs[e]:offs[e + 1]] // k
        assert np.all(np.diff(rows) > 0)
    if S:
        assert counts[E] == T and offs[E] == T * k


def test_dispatch_all_tokens_same_experts():
    T, E, k = 20, 8, 3
    idx = np.tile(np.array([5, 1, 6], np.int32), (T, 1))
    d = oracle.dispatch(_tiny(E, k, T=T), idx)
    assert d["counts"][5] == d["counts"][1] == d["counts"][6] == T
    assert d["counts"].sum() == T * k


def test_dispatch_rejects_bad_indices():
    w = _tiny(4, 2, T=2)
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(w, np.array([[0, 4], [1, 2]], np.int32))
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(w, np.array([[0, 1], [2, 2]], np.int32))
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(w, np.array([[-1, 1], [2, 3]], np.int32))


# ---------------------------------------------------------------- experts and the layer

def _dense_swiglu_torch(x, w1, w2):
    """Textbook SwiGLU FFN in torch fp64: (silu(x Wg^T) * (x Wu^T)) Wd^T."""
    F = w2.shape[1]
    x = torch.from_numpy(np.asarray(x, np.float64))
    w1 = torch.from_numpy(np.asarray(w1, np.float64))
    w2 = torch.from_numpy(np.asarray(w2, np.float64))
    h = torch.nn.functional.silu(x @ w1[:F].T) * (x @ w1[F:].T)
    return (h @ w2.T).numpy()


def _as_f64(a, mode):
    return synth.bf16_to_f32(a).astype(np.float64) if mode == "bf16" else a.astype(np.float64)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_single_expert_is_dense_swiglu(mode):
    w = Workload("one", 31, mode, 12, 64, 1, 1, 96, 0, "softmax")
    inp = synth.make_inputs(w)
    y, idx, g = oracle.layer(inp)
    assert np.all(idx == 0) and np.all(g == 1.0)
    ref = _dense_swiglu_torch(_as_f64(inp["x"], mode), _as_f64(inp["w1"][0], mode), _as_f64(inp["w2"][0], mode))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_identical_experts_plus_shared_is_two_dense_ffns(mode):
    w = Workload("same", 32, mode, 10, 64, 6, 3, 64, 1, "softmax")
    inp = synth.make_inputs(w)
    inp["w1"][:w.E] = inp["w1"][0]
    inp["w2"][:w.E] = inp["w2"][0]
    y, _, g = oracle.layer(inp)
    x = _as_f64(inp["x"], mode)
    routed = _dense_swiglu_torch(x, _as_f64(inp["w1"][0], mode), _as_f64(inp["w2"][0], mode))
    shared = _dense_swiglu_torch(x, _as_f64(inp["w1"][w.E], mode), _as_f64(inp["w2"][w.E], mode))
    # gates sum to 1 only up to fp32 rounding of each gate
    np.testing.assert_allclose(y, routed * g.astype(np.float64).sum(1, keepdims=True) + shared, rtol=1e-10,
                               atol=1e-10)


def test_layer_equals_gate_weighted_sum_of_experts():
    w = Workload("sum", 33, "bf16", 9, 64, 8, 3, 64, 1, "sigmoid", zipf_alpha=0.25)
    inp = synth.make_inputs(w)
    y, idx, g = oracle.layer(inp)
    x = _as_f64(inp["x"], "bf16")
    for t in range(w.T):
        ref = _dense_swiglu_torch(x[t:t + 1], _as_f64(inp["w1"][w.E], "bf16"), _as_f64(inp["w2"][w.E], "bf16"))[0]
        for j in range(w.k):
            e = idx[t, j]
            ref = ref + float(g[t, j]) * _dense_swiglu_torch(
                x[t:t + 1], _as_f64(inp["w1"][e], "bf16"), _as_f64(inp["w2"][e], "bf16"))[0]
        np.testing.assert_allclose(y[t], ref, rtol=1e-10, atol=1e-12)


def test_zero_gate_weights_give_zero_output():
    w = Workload("zg", 34, "bf16", 8, 64, 4, 2, 64, 1, "softmax")
    inp = synth.make_inputs(w, zero_gate=True)
    y, _, _ = oracle.layer(inp)
    assert np.all(y == 0.0)


def test_scaling_down_projection_scales_output():
    w = Workload("sc", 35, "f32", 8, 64, 4, 2, 64, 1, "softmax")
    inp = synth.make_inputs(w)
    y1, _, _ = oracle.layer(inp)
    inp2 = dict(inp, w2=inp["w2"] * np.float32(4.0))
    y2, _, _ = oracle.layer(inp2)
    np.testing.assert_array_equal(y2, 4.0 * y1)


def test_token_permutation_and_expert_relabelling():
    w = Workload("perm", 36, "f32", 16, 64, 8, 2, 64, 0, "softmax")
    inp = synth.make_inputs(w)
    y, idx, _ = oracle.layer(inp)
    p = np.random.default_rng(0).permutation(w.T)
    yp, _, _ = oracle.layer(dict(inp, x=np.ascontiguousarray(inp["x"][p])))
    np.testing.assert_array_equal(yp, y[p])
    q = np.random.default_rng(1).permutation(w.E)  # new expert e' = position of old expert in q
    inp_q = dict(inp, w_router=np.ascontiguousarray(inp["w_router"][q]),
                 w1=np.ascontiguousarray(inp["w1"][q]), w2=np.ascontiguousarray(inp["w2"][q]))
    yq, idxq, _ = oracle.layer(inp_q)
    np.testing.assert_array_equal(q[idxq], idx)
    np.testing.assert_allclose(yq, y, rtol=1e-12, atol=1e-14)


def test_layer_with_given_routing_uses_it():
    w = Workload("given", 37, "bf16", 6, 64, 8, 2, 64, 0, "softmax")
    inp = synth.make_inputs(w)
    idx = np.array([[7, 0]] * w.T, np.int32)
    gates = np.array([[0.25, 0.75]] * w.T, np.float32)
    y, iu, gu = oracle.layer(inp, idx=idx, gates=gates)
    np.testing.assert_array_equal(iu, idx)
    x = _as_f64(inp["x"], "bf16")
    ref = 0.25 * _dense_swiglu_torch(x, _as_f64(inp["w1"][7], "bf16"), _as_f64(inp["w2"][7], "bf16")) + \
        0.75 * _dense_swiglu_torch(x, _as_f64(inp["w1"][0], "bf16"), _as_f64(inp["w2"][0], "bf16"))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_fp8_mxfp4_expert_matches_independent_dequantised_ffn():
    """FP8 x MXFP4 expert: torch fp64 matmuls on independently dequantised operands.

    Weights: e2m1 values from the OCP table times 2^(e8m0-127). Activations and h:
    e4m3 codes from torch's float8 cast of v / 2^e with the power-of-two block scale.
    """
    w = Workload("fp8", 38, "fp8_mxfp4", 5, 256, 1, 1, 256, 0, "softmax")
    inp = synth.make_inputs(w)
    lut = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])

    def deq_w(codes, scales):
        nib = np.stack([codes & 15, codes >> 4], -1).reshape(codes.shape[0], -1)
        return lut[nib] * np.exp2(np.repeat(scales.astype(np.int64) - 127, 32, axis=-1))

    def q_torch(v):
        v = np.asarray(v, np.float32).reshape(-1, 128)
        amax = np.abs(v).max(1).astype(np.float64)
        e = np.array([oracle.e4m3_block_exponent(float(a)) for a in amax])
        sc = np.exp2(e)
        c = torch.from_numpy((v / sc[:, None]).astype(np.float32)).to(torch.float8_e4m3fn)
        return (c.to(torch.float64).numpy() * sc[:, None]).reshape(-1)

    W1 = deq_w(inp["w1"][0], inp["w1_scale"][0])
    W2 = deq_w(inp["w2"][0], inp["w2_scale"][0])
    y, _, _ = oracle.layer(inp)
    F = w.F
    for t in range(w.T):
        xq = q_torch(synth.bf16_to_f32(inp["x"][t]))
        u = torch.from_numpy(W1) @ torch.from_numpy(xq)
        h = (torch.nn.functional.silu(u[:F]) * u[F:]).numpy()
        hq = q_torch(h.astype(np.float32))
        ref = W2 @ hq
        np.testing.assert_allclose(y[t], ref, rtol=1e-10, atol=1e-12)


def test_integer_grid_layer_is_exact_in_fp64():
    """Integer inputs: router logits and expert pre-activations are exact integers."""
    w = Workload("grid", 39, "bf16", 8, 64, 4, 2, 64, 0, "softmax")
    inp = synth.make_inputs(w, grid=True)
    r = oracle.route(inp)
    x = _as_f64(inp["x"], "bf16")
    np.testing.assert_array_equal(r["logits"], x @ _as_f64(inp["w_router"], "bf16").T)


def test_golden_routing_examples():
    """Hand-worked routing cases (tests/golden/routing_examples.json)."""
    with open(os.path.join(GOLDEN, "routing_examples.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        logits = np.array([case["logits"]], np.float32)
        E = logits.shape[1]
        w = _tiny(E, case["k"], T=1, d=4, gating=case["gating"])
        bias = np.array(case["bias"], np.float32) if case.get("bias") else None
        r = oracle.route(_route_inputs(w, logits, bias))
        assert list(r["idx"][0]) == case["idx"], case["name"]
        np.testing.assert_allclose(r["gates"][0], case["gates"], rtol=2e-7, err_msg=case["name"])


def test_vectorised_e4m3_reference_matches_the_oracle_encoder():
    """tests/e4m3_ref.py (used for the exhaustive GPU conversion check) equals the oracle's
    per-value encoder on every code value, every midpoint, their fp32 neighbours, values
    past the saturation point and a seeded sample of fp32 patterns."""
    import e4m3_ref

    vals = np.array([oracle.e4m3_decode(c) for c in range(0x7F)], dtype=np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0
    pts = np.concatenate([vals, mids, [448.0, 449.0, 464.0, 480.0, 1e4, 3e38, 1e-30, 1e-45]]).astype(np.float32)
    bits = pts.view(np.uint32)
    nb = np.concatenate([bits, bits + 1, bits - 1, np.array([0, 1], dtype=np.uint32)])
    nb = nb[(nb & 0x7F800000) != 0x7F800000]
    rng = np.random.default_rng(5)
    sample = rng.integers(0, 0x43E00001, size=20000, dtype=np.uint32)
    allbits = np.concatenate([nb, sample, sample | 0x80000000, nb | 0x80000000])
    got = e4m3_ref.encode_bits(allbits)
    want = np.array([oracle.e4m3_encode(float(v)) for v in allbits.view(np.float32)], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("mode", ["fp8_mxfp4", "bf16"])
def test_down_rows_is_linear2(mode):
    """oracle.down_rows: torch fp64 matmul on independently dequantised W2 (FP8 x MXFP4: the
    OCP e2m1 table times 2^(e8m0 - 127)); integer rows and integer weights give exact sums."""
    w = Workload("down", 41, mode, 4, 256, 3, 1, 256, 1, "softmax")
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(3)
    hhat = rng.standard_normal((5, w.F))
    if mode == "fp8_mxfp4":
        lut = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
        codes, scales = inp["w2"][2], inp["w2_scale"][2]
        nib = np.stack([codes & 15, codes >> 4], -1).reshape(codes.shape[0], -1)
        W2 = lut[nib] * np.exp2(np.repeat(scales.astype(np.int64) - 127, 32, axis=-1))
    else:
        W2 = _as_f64(inp["w2"][2], "bf16")
    got = oracle.down_rows(inp, 2, hhat)
    np.testing.assert_allclose(got, (torch.from_numpy(hhat) @ torch.from_numpy(W2).T).numpy(), rtol=1e-11,
                               atol=1e-12)
    g = synth.make_inputs(w, grid=True)
    hi = rng.integers(-3, 4, size=(3, w.F)).astype(np.float64)
    W2g = _as_f64(g["w2"][1], "bf16") if mode == "bf16" else None
    if mode == "bf16":
        np.testing.assert_array_equal(oracle.down_rows(g, 1, hi), hi @ W2g.T)
    # the expert on an input row equals linear2 of its quantised h (FP8) or of h
    xin = oracle.input_rows(inp, [1])
    out, h = oracle.expert_rows(inp, 0, xin, want_h=True)
    if mode == "fp8_mxfp4":
        c, s = oracle.quant_e4m3_b128(h.astype(np.float32))
        hq = np.array([oracle.e4m3_decode(int(v)) for v in c.reshape(-1)]).reshape(c.shape) * np.repeat(s, 128, 1)
    else:
        hq = h
    np.testing.assert_array_equal(oracle.down_rows(inp, 0, hq), out)


# ---------------------------------------------------------------- capacity variant and bias update

def _brute_capacity(idx, E, S, capacity):
    """Per expert, its slots in slot order; the first `capacity` kept."""
    T, k = idx.shape
    slots = {e: [s for s in range(T * k) if idx.reshape(-1)[s] == e] for e in range(E)}
    kept = {e: v[:capacity] for e, v in slots.items()}
    drop = {e: v[capacity:] for e, v in slots.items()}
    return kept, drop


@pytest.mark.parametrize("T,E,k,S,cap", [(40, 8, 2, 1, 7), (33, 6, 3, 0, 10), (50, 16, 4, 1, 0), (21, 5, 5, 1, 4),
                                         (64, 8, 2, 0, 1000)])
def test_capacity_dispatch_brute_force(T, E, k, S, cap):
    w = _tiny(E, k, T=T, S=S)
    rng = np.random.default_rng(T * 7 + E)
    p = rng.dirichlet(np.full(E, 0.4))
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    r = oracle.dispatch_capacity(w, idx, cap)
    kept, drop = _brute_capacity(idx, E, S, cap)
    nk = np.array([len(kept[e]) for e in range(E)])
    nd = np.array([len(drop[e]) for e in range(E)])
    np.testing.assert_array_equal(r["counts"][:E], nk)
    np.testing.assert_array_equal(r["dropped"], nd)
    assert np.all(nk <= cap) and nk.sum() + nd.sum() == T * k
    D = nd.sum()
    assert r["offsets"][0] == D and r["offsets"][E] == T * k
    np.testing.assert_array_equal(np.diff(r["offsets"][: E + 1]), nk)
    if S:
        assert r["counts"][E] == T and r["offsets"][E + 1] == T * k + T
    # kept rows: expert by expert, in slot order; dropped rows 0..D-1 likewise
    exp_r2s = [s for e in range(E) for s in drop[e]] + [s for e in range(E) for s in kept[e]]
    np.testing.assert_array_equal(r["row_to_slot"], np.array(exp_r2s, dtype=np.int32))
    s2r = np.full(T * k, -1, dtype=np.int32)
    for row, s in enumerate(exp_r2s):
        if row >= D:
            s2r[s] = row
    np.testing.assert_array_equal(r["slot_to_row"], s2r)
    assert sorted(r["row_to_slot"].tolist()) == list(range(T * k))
    if cap >= max(np.bincount(idx.reshape(-1), minlength=E)):
        d = oracle.dispatch(w, idx)  # nothing dropped: the dropless dispatch
        for key in ("counts", "offsets", "slot_to_row", "row_to_slot"):
            np.testing.assert_array_equal(r[key], d[key])


def test_dropping_layer_closed_forms():
    """Keeping every slot is the layer; dropping a slot equals giving it gate 0; dropping all
    leaves the shared expert, a dense SwiGLU FFN."""
    w = Workload("drop", 61, "bf16", 12, 64, 6, 3, 64, 1, "softmax")
    inp = synth.make_inputs(w)
    y, idx, gates = oracle.layer(inp)
    keep = np.ones_like(idx, dtype=np.uint8)
    np.testing.assert_array_equal(oracle.layer_dropping(inp, idx, gates, keep), y)
    rng = np.random.default_rng(1)
    keep = (rng.random(idx.shape) < 0.6).astype(np.uint8)
    g0 = np.where(keep == 1, gates, 0.0).astype(np.float32)
    y0, _, _ = oracle.layer(inp, idx=idx, gates=g0)
    np.testing.assert_array_equal(oracle.layer_dropping(inp, idx, gates, keep), y0)
    none = oracle.layer_dropping(inp, idx, gates, np.zeros_like(keep))
    x = _as_f64(inp["x"], "bf16")
    ref = _dense_swiglu_torch(x, _as_f64(inp["w1"][w.E], "bf16"), _as_f64(inp["w2"][w.E], "bf16"))
    np.testing.assert_allclose(none, ref, rtol=1e-12, atol=1e-13)


def test_bias_update_closed_forms():
    E = 8
    b = np.linspace(-0.3, 0.4, E).astype(np.float32)
    np.testing.assert_array_equal(oracle.bias_update(np.full(E, 5), b, 0.01), b)  # on target
    c = np.zeros(E, dtype=np.int32)
    c[3] = 40
    got = oracle.bias_update(c, b, 0.125)
    want = b + np.float32(0.125)
    want[3] = b[3] - np.float32(0.125)
    np.testing.assert_array_equal(got, want)
    c = np.array([3, 5, 4, 4, 4, 4, 4, 4], dtype=np.int32)  # mean 4: experts 2..7 exactly on target
    got = oracle.bias_update(c, np.zeros(E, np.float32), 0.5)
    np.testing.assert_array_equal(got, np.array([0.5, -0.5, 0, 0, 0, 0, 0, 0], dtype=np.float32))


def test_bias_update_loop_balances_a_skewed_router():
    """The MoE lesson's loop (Step 2: 100 tokens routed, then +-gamma per expert, repeated):
    on a router skewed towards a few experts the per-expert load moves towards uniform."""
    w = Workload("loop", 62, "f32", 100, 32, 8, 2, 128, 0, "softmax")
    inp = synth.make_inputs(w)
    # skew: scale up the router rows of experts 0 and 1
    inp["w_router"][:2] *= 4.0
    bias = np.zeros(w.E, dtype=np.float32)
    loads = []
    for _ in range(50):
        inp["bias"] = bias
        r = oracle.route(inp)
        counts = oracle.dispatch(w, r["idx"])["counts"]
        loads.append(counts.max() / counts.mean())
        bias = oracle.bias_update(counts, bias, 0.05)
    assert loads[0] > 1.5, loads[0]
    assert max(loads[-10:]) <= 1.2 and max(loads[-10:]) < loads[0] - 0.3, loads


def test_fp8_row_generator_encodes_within_half_step():
    """synth.fp8_rows: the scale is 2^(floor(log2 amax) - 8) per 128 values, and each code is
    torch's e4m3 cast of value / scale (round to nearest even; saturated at 448)."""
    codes, scales = synth.fp8_rows(5, 9, 6, 256, 0.3)
    z = synth.normal(5, 9, (6, 256), 0.3)  # the very draws (same seed, tensor, counters)
    for r in range(6):
        for b in range(2):
            v = z[r, b * 128:(b + 1) * 128]
            e = math.floor(math.log2(float(np.abs(v).max()))) - 8
            assert scales[r, b] == np.float32(2.0 ** e)
            want = torch.from_numpy((v / scales[r, b]).astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
            np.testing.assert_array_equal(codes[r, b * 128:(b + 1) * 128], want.view(torch.uint8).numpy())
    gc, gs = synth.fp8_rows(5, 9, 4, 128, 0.0, grid=(-3, 3))
    vals = np.array([oracle.e4m3_decode(int(c)) for c in gc.reshape(-1)]).reshape(gc.shape)
    np.testing.assert_array_equal(vals, synth.intgrid(5, 9, (4, 128), -3, 3))
    assert np.all(gs == 1.0)


def test_dense_fp8_mxfp4_gemm():
    """oracle.gemm_fp8_mxfp4: torch fp64 matmul on independently dequantised operands (torch's
    float8 decode of the A codes; the OCP e2m1 table times 2^(e8m0 - 127) for B); integer
    operands give exact integer sums; and linear2 of the layer is this GEMM on h."""
    a, a_s = synth.fp8_rows(3, 1, 7, 256, 1.0)
    b, b_s = synth.mxfp4(3, 2, 1, 64, 256, 0.1)
    b, b_s = b[0], b_s[0]
    lut = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    nib = np.stack([b & 15, b >> 4], -1).reshape(b.shape[0], -1)
    B = lut[nib] * np.exp2(np.repeat(b_s.astype(np.int64) - 127, 32, axis=-1))
    A = torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float64).numpy() * np.repeat(a_s, 128, 1)
    np.testing.assert_array_equal(oracle.dequant_e4m3_rows(a, a_s), A)
    np.testing.assert_allclose(oracle.gemm_fp8_mxfp4(a, a_s, b, b_s), A @ B.T, rtol=1e-12, atol=1e-12)
    gi, gs = synth.fp8_rows(3, 3, 5, 128, 0.0, grid=(-3, 3))
    wb, ws_ = synth.mxfp4(3, 4, 1, 16, 128, 0.0, grid=(-2, 2))
    want = synth.intgrid(3, 3, (5, 128), -3, 3).astype(np.int64) @ \
        synth.intgrid(3, 4, (16, 128), -2, 2).astype(np.int64).T
    np.testing.assert_array_equal(oracle.gemm_fp8_mxfp4(gi, gs, wb[0], ws_[0]), want.astype(np.float64))


def test_fp8_fp8_expert_matches_independent_dequantised_ffn():
    """FP8 e4m3 x e4m3 expert: torch fp64 matmuls on operands dequantised with torch's float8
    decode times the 1x128 scales; activations and h through torch's float8 cast of v / 2^e."""
    w = Workload("fp8x8", 42, "fp8_fp8", 4, 256, 2, 1, 256, 1, "softmax")
    inp = synth.make_inputs(w)

    def deq(codes, scales):
        return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * \
            np.repeat(scales.astype(np.float64), 128, axis=-1)

    def q_torch(v):
        v = np.asarray(v, np.float32).reshape(-1, 128)
        amax = np.abs(v).max(1).astype(np.float64)
        e = np.array([oracle.e4m3_block_exponent(float(a)) for a in amax])
        sc = np.exp2(e)
        c = torch.from_numpy((v / sc[:, None]).astype(np.float32)).to(torch.float8_e4m3fn)
        return (c.to(torch.float64).numpy() * sc[:, None]).reshape(-1)

    idx = np.zeros((w.T, 1), np.int32)
    idx[1::2] = 1
    gates = np.ones((w.T, 1), np.float32)
    y, _, _ = oracle.layer(inp, idx=idx, gates=gates)
    F = w.F
    for t in range(w.T):
        xq = q_torch(synth.bf16_to_f32(inp["x"][t]))
        out = np.zeros(w.d)
        for g in (int(idx[t, 0]), w.E):
            W1 = deq(inp["w1"][g], inp["w1_scale"][g])
            W2 = deq(inp["w2"][g], inp["w2_scale"][g])
            u = torch.from_numpy(W1) @ torch.from_numpy(xq)
            h = (torch.nn.functional.silu(u[:F]) * u[F:]).numpy()
            out += W2 @ q_torch(h.astype(np.float32))
        np.testing.assert_allclose(y[t], out, rtol=1e-10, atol=1e-12)
    # integer-grid e4m3 weights (scale 1) and integer activations: exact pre-activations
    g = synth.make_inputs(w, grid=True)
    xin = oracle.input_rows(g, [0])
    _, h = oracle.expert_rows(g, 0, xin, want_h=True)
    W1 = synth.intgrid(w.seed, synth.TID_W1, (w.G * 2 * F, w.d), -2, 2).reshape(w.G, 2 * F, w.d)[0]
    u = W1.astype(np.float64) @ xin[0]
    assert np.all(u == np.round(u))  # integer pre-activations, exact in fp64
    np.testing.assert_allclose(h[0], u[:F] / (1.0 + np.exp(-u[:F])) * u[F:], rtol=1e-15, atol=0)
