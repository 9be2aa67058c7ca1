"""A vectorised fp32 -> e4m3 (OCP E4M3FN) round-to-nearest-even encoder over fp32 bit
patterns, for exhaustive comparisons that the oracle's per-value encoder is too slow for.

It is built from the oracle's own decoder table: the 127 non-negative finite codes in
ascending order and the midpoints between neighbours (each exactly representable in
fp32, as e4m3 values carry four significant bits).  A magnitude below a code's upper
midpoint rounds down to it, one above rounds up, one exactly on a midpoint goes to the
even code, and magnitudes beyond 448 saturate to 448 (code 0x7E).  The sign bit is
copied.  tests/test_oracle.py pins it to oracle.e4m3_encode.
"""
from __future__ import annotations

import numpy as np

import oracle

_MID_BITS = None


def _mid_bits() -> np.ndarray:
    global _MID_BITS
    if _MID_BITS is None:
        vals = np.array([oracle.e4m3_decode(c) for c in range(0x7F)], dtype=np.float64)
        assert np.all(np.diff(vals) > 0)
        mids = (vals[:-1] + vals[1:]) / 2.0
        assert np.all(mids.astype(np.float32).astype(np.float64) == mids)
        _MID_BITS = mids.astype(np.float32).view(np.uint32)
    return _MID_BITS


def encode_bits(bits: np.ndarray) -> np.ndarray:
    """fp32 bit patterns (uint32, finite values) -> e4m3 codes (uint8)."""
    mids = _mid_bits()
    bits = np.asarray(bits, dtype=np.uint32)
    mag = bits & np.uint32(0x7FFFFFFF)
    i = np.searchsorted(mids, mag, side="left")  # midpoints strictly below
    on_mid = mids[np.minimum(i, mids.size - 1)] == mag
    code = i + (on_mid & (i % 2 == 1))  # on a midpoint between i and i + 1: the even one
    sign = ((bits >> np.uint32(24)) & np.uint32(0x80)).astype(np.int64)
    return (code.astype(np.int64) | sign).astype(np.uint8)


def decode_codes(codes: np.ndarray) -> np.ndarray:
    """e4m3 codes -> fp64 values (the oracle's decoder, tabulated)."""
    table = np.array([oracle.e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]
