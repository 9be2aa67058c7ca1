"""The capacity variant (expert capacity with token dropping) and the aux-loss-free bias
update on the GPU, through the C ABI, against the oracle: the kept and dropped slots, counts,
offsets and both permutations bit for bit; the layer on the kept slots within the mode's
tolerance; the bias update bit for bit, alone and inside a route -> dispatch -> update loop."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_dispatch_amd as moe
import oracle
import synth
from synth import Workload
from moe_testlib import TOL, cfg_of, check_xq, log, rel_l2, to_f64, upload

pytestmark = pytest.mark.gpu

CASES = [
    Workload("cap_bf16_multi", 5001, "bf16", 700, 256, 64, 6, 256, 1, "sigmoid", zipf_alpha=0.5),
    Workload("cap_fp8_multi", 5002, "fp8_mxfp4", 600, 256, 32, 4, 256, 1, "softmax", zipf_alpha=1.0),
    Workload("cap_bf16_one_block", 5003, "bf16", 100, 128, 16, 2, 128, 0, "softmax", zipf_alpha=1.0),
    Workload("cap_f32", 5004, "f32", 90, 128, 8, 3, 128, 1, "sigmoid", zipf_alpha=0.5),
]


def _check_capacity_dispatch(w, idx, d, cfg, ws, cap):
    got = moe.dispatch_capacity(cfg, idx, cap, d["x"] if w.mode == "fp8_mxfp4" else None, ws=ws)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 0
    ref = oracle.dispatch_capacity(w, idx.cpu().numpy(), cap)
    for key in ("counts", "dropped", "offsets", "slot_to_row", "row_to_slot"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=f"{key} at capacity {cap}")
    return got, ref


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_capacity_dispatch_and_layer(w):
    log(f"case {w.name}: mode={w.mode} T={w.T} E={w.E} k={w.k}")
    inp = synth.make_inputs(w)
    d = upload(inp)
    cfg = cfg_of(w)
    ws = moe.alloc_workspace(cfg)
    idx, gate, _, _ = moe.route(cfg, d["x"], d["w_router"], d["bias"], ws=ws)
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.E)
    for factor in (0.0, 0.5, 1.0, 1.25, float(counts.max()) * w.E / (w.T * w.k)):
        cap = moe.capacity_of(factor, cfg)
        got, ref = _check_capacity_dispatch(w, idx, d, cfg, ws, cap)
        if w.mode == "fp8_mxfp4":
            check_xq(w, inp, got["xq"], got["xq_scale"])
        if cap >= counts.max():
            plain = moe.dispatch(cfg, idx, d["x"], ws=ws)
            for key in ("counts", "offsets", "slot_to_row", "row_to_slot"):
                assert torch.equal(plain[key], got[key]), key
        # the layer on the kept slots: ffn and combine run unchanged
        yp = moe.ffn(cfg, d["w1"], d["w2"], d["w1_scale"], d["w2_scale"], x=None if w.mode == "fp8_mxfp4" else d["x"],
                     xq=got["xq"], xq_scale=got["xq_scale"], offsets=got["offsets"],
                     row_to_slot=got["row_to_slot"], ws=ws)
        y = moe.combine(cfg, yp, got["slot_to_row"], gate)
        torch.cuda.synchronize()
        keep = (got["slot_to_row"].cpu().numpy() >= 0).reshape(w.T, w.k)
        y_ref = oracle.layer_dropping(inp, idx.cpu().numpy(), gate.cpu().numpy(), keep)
        y_gpu = to_f64(y)
        assert np.all(np.isfinite(y_gpu))
        if np.linalg.norm(y_ref) == 0:
            assert np.all(y_gpu == 0)
            err = 0.0
        else:
            err = rel_l2(y_gpu, y_ref)
        assert err <= TOL[w.mode], f"capacity {cap}: rel L2 {err:.3e}"
        log(f"  capacity {cap}: dropped {int(ref['dropped'].sum())} of {w.T * w.k} slots, rel L2 {err:.2e}")


def test_bias_update_bit_exact():
    E = 256
    cfg = moe.Config(T=1000, d=128, E=E, k=8, F=128, n_shared=1, gating="sigmoid")
    rng = np.random.default_rng(9)
    for trial in range(4):
        counts = rng.poisson(31.25, size=E + 1).astype(np.int32)
        if trial == 1:
            counts[:E] = 7  # every expert on target
        if trial == 2:
            counts[:E] = 0
            counts[5] = 8000
        bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
        b = torch.from_numpy(bias).cuda()
        moe.bias_update(cfg, torch.from_numpy(counts).cuda(), b, 0.001 * (trial + 1))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(b.cpu().numpy(), oracle.bias_update(counts[:E], bias, 0.001 * (trial + 1)))


def test_bias_update_loop_on_device():
    """route -> dispatch -> bias update, repeated on the device with a skewed router: each
    update equals the oracle's from the GPU's counts, each selection equals the oracle's top-k
    over the GPU's keys, and the load moves towards uniform."""
    w = Workload("loop", 5005, "bf16", 512, 256, 32, 4, 128, 1, "sigmoid")
    inp = synth.make_inputs(w)
    inp["w_router"][:4] = synth.f32_to_bf16(synth.bf16_to_f32(inp["w_router"][:4]) * 4.0)
    d = upload(inp)
    cfg = cfg_of(w)
    ws = moe.alloc_workspace(cfg)
    bias = torch.zeros(w.E, dtype=torch.float32, device="cuda")
    loads = []
    for it in range(30):
        b_before = bias.cpu().numpy()
        idx, gate, logits, keys = moe.route(cfg, d["x"], d["w_router"], bias, ws=ws, want_logits=True)
        dsp = moe.dispatch(cfg, idx, None, ws=ws)
        moe.bias_update(cfg, dsp["counts"], bias, 0.01)
        torch.cuda.synchronize()
        assert moe.read_device_error(cfg, ws) == 0
        o_idx, _ = oracle.topk_gates_from(w, logits.cpu().numpy(), keys.cpu().numpy())
        np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
        c = dsp["counts"].cpu().numpy()
        np.testing.assert_array_equal(bias.cpu().numpy(), oracle.bias_update(c[: w.E], b_before, 0.01))
        loads.append(c[: w.E].max() / c[: w.E].mean())
    log(f"load max/mean: first {loads[0]:.2f}, last {loads[-1]:.2f}")
    assert loads[0] > 1.5 and max(loads[-5:]) < loads[0] - 0.3, loads
