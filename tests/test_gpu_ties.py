"""GPU routing on inputs built to tie: the tie rule of top-k (equal keys go to the lower
expert index) and the bounded-wait give-up path of the persistent kernel.

Ties.  Integer-grid activations and router rows make every logit an exact integer on
both sides (each fp32 partial sum is exact), and router rows repeated across experts
give several experts the very same logit for every token; a zero router row gives
logit +0, and integer biases (some of them -0.0) give many exactly equal keys, zeros
included.  With bit-identical logits and softmax gating the keys are bit-identical on
both sides, so the oracle's top-k from its own logits must equal the GPU's on every
token; with sigmoid gating the GPU's exported keys decide (the oracle's top-k over
them must equal the GPU's choice).  Dispatch of the tied choices is checked bit for bit
as well, and the persistent kernel must give the step chain's bits.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_dispatch_amd as moe
import oracle
import synth
from synth import Workload
from moe_testlib import cfg_of, check_dispatch, check_outputs, check_routing, log, upload

pytestmark = pytest.mark.gpu


def tie_inputs(w: Workload, dup_every: int = 3):
    """Integer-grid inputs whose router rows repeat (experts e-1 and e share a row when
    e % dup_every == 1), with a zero row for the last expert and integer selection biases."""
    inp = synth.make_inputs(w, grid=True)
    wr = inp["w_router"].copy()
    for e in range(1, w.E, dup_every):
        wr[e] = wr[e - 1]
    wr[w.E - 1] = 0
    inp["w_router"] = wr
    rng = np.random.default_rng(w.seed)
    if w.gating == "softmax":
        b = rng.integers(-3, 4, size=w.E).astype(np.float32)
    else:
        b = (rng.integers(-1, 2, size=w.E) * 0.5).astype(np.float32)
    b[b == 0] = -0.0
    b[: w.E // 4] = 0.0
    inp["bias"] = b
    return inp


def tied_tokens(keys: np.ndarray, k: int) -> int:
    """Tokens whose k-th largest key equals another key (a tie decided by the rule)."""
    srt = -np.sort(-keys, axis=1)
    kth = srt[:, k - 1:k]
    return int(((keys == kth).sum(axis=1) > 1).sum())


CASES = [
    Workload("tie_bf16_e8_softmax", 4001, "bf16", 300, 256, 8, 2, 128, 0, "softmax"),
    Workload("tie_bf16_e64_softmax", 4002, "bf16", 257, 256, 64, 6, 128, 1, "softmax"),
    Workload("tie_bf16_e256_softmax", 4003, "bf16", 300, 256, 256, 8, 128, 1, "softmax"),
    Workload("tie_bf16_e256_sigmoid", 4004, "bf16", 300, 256, 256, 8, 128, 1, "sigmoid"),
    Workload("tie_bf16_e64_sigmoid", 4005, "bf16", 130, 128, 64, 4, 128, 0, "sigmoid"),
    Workload("tie_f32_e8_softmax", 4006, "f32", 200, 128, 8, 3, 128, 0, "softmax"),
    Workload("tie_fp8_e64_softmax", 4007, "fp8_mxfp4", 150, 256, 64, 8, 256, 1, "softmax"),
    # the tiled router (E a multiple of 256, T >= 2048)
    Workload("tie_bf16_e256_tiled", 4008, "bf16", 2100, 256, 256, 8, 128, 1, "softmax"),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_ties_go_to_the_lower_expert(w):
    log(f"case {w.name}: T={w.T} d={w.d} E={w.E} k={w.k} {w.gating} mode={w.mode}")
    inp = tie_inputs(w)
    d = upload(inp)
    cfg = cfg_of(w)
    ws = moe.alloc_workspace(cfg)
    idx, gate, logits, keys = moe.route(cfg, d["x"], d["w_router"], d["bias"], ws=ws, want_logits=True)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 0
    ref = oracle.route(inp)
    np.testing.assert_array_equal(logits.cpu().numpy(), ref["logits"], err_msg="integer-grid logits")
    ky = keys.cpu().numpy()
    n_tied = tied_tokens(ky, w.k)
    assert n_tied >= w.T // 10, f"only {n_tied} tokens with a tie at the k-th key"
    if w.gating == "softmax":
        # identical keys on both sides: the oracle's own routing, bit for bit
        np.testing.assert_array_equal(ky, ref["keys"], err_msg="keys")
        np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"], err_msg="top-k with ties")
    check_routing(w, inp, idx, gate, logits, keys)
    dsp = moe.dispatch(cfg, idx, d["x"], ws=ws)
    check_dispatch(w, idx, dsp)
    # the whole layer on the tied routing, and the persistent kernel's bits
    y, r = moe.layer_unfused(cfg, d["x"], d["w_router"], d["w1"], d["w2"], d["w1_scale"], d["w2_scale"], d["bias"],
                             ws=ws)
    assert torch.equal(r["topk_idx"], idx)
    check_outputs(w, inp, y, idx, gate, np.arange(w.T))
    y2 = moe.layer_fused(cfg, d["x"], d["w_router"], d["w1"], d["w2"], d["w1_scale"], d["w2_scale"], d["bias"],
                         ws=ws)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 0
    view = torch.int32 if w.mode == "f32" else torch.int16
    assert torch.equal(y2.view(view), y.view(view)), "fused != unfused"
    log(f"case {w.name}: {n_tied} of {w.T} tokens tied at the k-th key")


# ---- the bounded waits' give-up path ------------------------------------------------------

TIMEOUT_CASES = [
    Workload("timeout_bf16", 4101, "bf16", 200, 384, 64, 6, 256, 1, "sigmoid", zipf_alpha=0.25),
    Workload("timeout_fp8_decode", 4102, "fp8_mxfp4", 5, 512, 64, 8, 256, 1, "softmax"),
]


@pytest.mark.parametrize("w", TIMEOUT_CASES, ids=[c.name for c in TIMEOUT_CASES])
def test_given_up_waits_end_and_leave_clean_sync_words(w):
    """With the error word pre-set to MOE_DEVERR_TIMEOUT, every bounded wait of the
    persistent kernel gives up at once.  The launch must still end, report the code, and
    leave its synchronisation words zero: after clearing only the error word, the next
    launch must give the step chain's bits.  Every input is the same as the launch before,
    so each step that runs early rewrites the values already there (one dispatch block:
    no step updates a buffer in place), and no address depends on a half-written value."""
    log(f"case {w.name}: pre-set timeout")
    d = upload(synth.make_inputs(w))
    cfg = cfg_of(w)
    assert (w.T + 255) // 256 == 1
    ws = moe.alloc_workspace(cfg)
    y_ref, _ = moe.layer_unfused(cfg, d["x"], d["w_router"], d["w1"], d["w2"], d["w1_scale"], d["w2_scale"],
                                 d["bias"], ws=ws)
    args = (cfg, d["x"], d["w_router"], d["w1"], d["w2"], d["w1_scale"], d["w2_scale"], d["bias"])
    y1 = moe.layer_fused(*args, ws=ws)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 0
    view = torch.int32 if w.mode == "f32" else torch.int16
    assert torch.equal(y1.view(view), y_ref.view(view))
    word = ws.view(torch.int32)
    word[0] = 4  # MOE_DEVERR_TIMEOUT
    moe.layer_fused(*args, ws=ws)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 4
    word[0] = 0  # the error word only; the synchronisation words are the kernel's to clear
    y3 = moe.layer_fused(*args, ws=ws)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 0, "a wait expired after the give-up launch"
    assert torch.equal(y3.view(view), y_ref.view(view)), "stale synchronisation words after a give-up"
