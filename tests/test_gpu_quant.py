"""The FP8 quantiser on fp32 inputs (moe_quant_e4m3, the rule and conversion instructions
the linear1 epilogue applies to h): bit-exact against the oracle's rule on seeded fp32
rows with full 24-bit mantissas, and the conversion itself exhaustively over every fp32
pattern of magnitude at most 448 (the range a block-scaled value falls in)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_dispatch_amd as moe
import oracle
import e4m3_ref
from moe_testlib import log

pytestmark = pytest.mark.gpu


def test_quantiser_fp32_rows_match_the_oracle():
    rng = np.random.default_rng(11)
    rows, K = 1000, 1024
    # full-mantissa fp32 values over many magnitudes (block maxima on both sides of powers of two)
    v = (rng.standard_normal((rows, K)) * np.exp2(rng.integers(-30, 30, size=(rows, 1)))).astype(np.float32)
    v[3, :128] = 0.0            # an all-zero block
    v[4, :128] = 448.0          # a block exactly at the e4m3 maximum
    v[5, 5] = np.float32(448.0) * np.float32(2.0) ** -20  # a block maximum exactly 448 * 2^-20
    v[5, 6:128] = 1e-9
    v[6, :128] = np.float32(1e-40)  # fp32 subnormals
    codes, scales = moe.quant_e4m3(torch.from_numpy(v).cuda())
    torch.cuda.synchronize()
    oc, os_ = oracle.quant_e4m3_b128(v)
    np.testing.assert_array_equal(scales.cpu().numpy(), os_, err_msg="scales")
    np.testing.assert_array_equal(codes.cpu().numpy(), oc, err_msg="codes")


@pytest.mark.slow
def test_e4m3_conversion_every_fp32_pattern_up_to_448():
    """Each 128-value block holds 127 consecutive fp32 patterns and one 448.0, so its scale is
    1 and every pattern reaches the conversion unscaled.  All 2 x 1,138,753,537 patterns of
    magnitude <= 448 (both signs) are compared with the vectorised encoder pinned to the
    oracle's."""
    top = 0x43E00000  # 448.0
    per = 127
    chunk = per * (1 << 20)
    anchor = np.float32(448.0).view(np.uint32)
    bad_total = 0
    for sign in (0, 0x80000000):
        start = 0
        while start <= top:
            n = min(chunk, top + 1 - start)
            nblk = (n + per - 1) // per
            bits = np.arange(start, start + nblk * per, dtype=np.uint64)
            bits = np.minimum(bits, top).astype(np.uint32) | np.uint32(sign)
            blk = np.empty((nblk, 128), dtype=np.uint32)
            blk[:, :per] = bits.reshape(nblk, per)
            blk[:, per] = anchor
            dev = torch.from_numpy(blk.view(np.float32)).cuda()
            codes, scales = moe.quant_e4m3(dev)
            torch.cuda.synchronize()
            assert bool((scales == 1.0).all()), "a block's scale is not 1"
            got = codes.cpu().numpy()[:, :per].reshape(-1)
            want = e4m3_ref.encode_bits(bits)
            bad = np.nonzero(got != want)[0]
            if bad.size:
                b = bits[bad[:5]]
                log(f"mismatch at patterns {[hex(int(x)) for x in b]}: gpu {got[bad[:5]]} want {want[bad[:5]]}")
            bad_total += bad.size
            start += n
        log(f"sign {sign:#x}: done")
    assert bad_total == 0, f"{bad_total} fp32 patterns convert differently"
