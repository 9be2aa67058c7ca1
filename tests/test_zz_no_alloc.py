"""moe_dispatch_noalloc (the dispatch without a workspace) against moe_dispatch, through
the C ABI: bit-exact counts, offsets, both permutations and FP8 codes and scales, on two
calls in a row, the second with a smaller input (the fixed device scratch keeps the first
call's contents), and its error word."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_dispatch_amd as moe
import synth
from synth import Workload
from moe_testlib import cfg_of, log, upload

pytestmark = pytest.mark.gpu

KEYS = ("counts", "offsets", "slot_to_row", "row_to_slot", "xq", "xq_scale")


def _routing(w, seed):
    """Seeded top-k choices: k distinct experts per token, skewed towards a few experts."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(w.E, 0.3))
    idx = np.stack([rng.choice(w.E, size=w.k, replace=False, p=p) for _ in range(w.T)]).astype(np.int32)
    return torch.from_numpy(idx).cuda()


def _compare(w, d, idx):
    cfg = cfg_of(w)
    ws = moe.alloc_workspace(cfg)
    ref = moe.dispatch(cfg, idx, d["x"], ws=ws)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = moe.dispatch_noalloc(cfg, idx, d["x"], err=err)
    torch.cuda.synchronize()
    assert moe.read_device_error(cfg, ws) == 0 and int(err.item()) == 0
    for key in KEYS:
        if ref[key] is None:
            continue
        assert torch.equal(got[key], ref[key]), key


@pytest.mark.parametrize("mode", ["fp8_mxfp4", "bf16"])
def test_noalloc_dispatch_matches_dispatch(mode):
    big = Workload("noalloc_big", 3101, mode, 3000, 256, 64, 6, 128, 1, "softmax")
    small = Workload("noalloc_small", 3102, mode, 700, 256, 64, 6, 128, 1, "softmax")
    tiny = Workload("noalloc_tiny", 3103, mode, 100, 256, 64, 6, 128, 1, "softmax")
    for w in (big, small, tiny):
        log(f"noalloc dispatch {mode} T={w.T} E={w.E} k={w.k}")
        d = upload(synth.make_inputs(w))
        _compare(w, d, _routing(w, w.seed))


def test_noalloc_dispatch_reports_bad_indices_and_limits():
    w = Workload("noalloc_err", 3104, "bf16", 300, 128, 16, 2, 128, 0, "softmax")
    cfg = cfg_of(w)
    idx = _routing(w, 7)
    idx[5, 1] = w.E
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.dispatch_noalloc(cfg, idx, None, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 1  # MOE_DEVERR_INDEX
    # the block counts of (T + 255) / 256 * E > 262144 do not fit the fixed scratch
    huge = moe.Config(T=300000, d=128, E=256, k=2, F=128, mode="bf16")
    with pytest.raises(moe.MoeError) as ex:
        moe.dispatch_noalloc(huge, torch.zeros(huge.T, huge.k, dtype=torch.int32, device="cuda"), None)
    assert ex.value.status == 5
