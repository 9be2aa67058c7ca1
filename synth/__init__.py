"""Seeded synthetic inputs for the MoE-layer forward (host side).

This package only draws numbers; it holds none of the layer's arithmetic.  The
same arrays feed the CPU oracle and the GPU library.  All draws come from
Philox4x32-10 keyed by (config seed, tensor id); see ``synth.c``.

Workloads (sizes from the pages' model shapes and per-rank batch sizes):

* ``tiny_f32``       T=64,  d=128,  E=8,   k=2, F=256,   no shared, softmax, fp32
* ``mixtral_bf16``   T=4096, d=4096, E=8,  k=2, F=14336, no shared, softmax, bf16
* ``dsv3_bf16``      T=8192, d=7168, E=256, k=8, F=2048, 1 shared, sigmoid + Zipf bias, bf16
* ``dsv3_fp8fp4``    d=7168, E=256, k=8, F=2048, 1 shared, softmax, FP8 e4m3 x MXFP4,
                     T in {512, 8192, 32768}
* ``decode_fp8fp4``  the same layer and tensors (same seed), T in {1, 64}
* ``dsv3_fp8fp4_zipf`` the same layer and tensors with sigmoid scores and the Zipf bias
* ``dsv3_fp8fp8``    the same shape with FP8 e4m3 weights (1x128 power-of-two scales), T = 8192
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

U64, U32, I32, F32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_float
VP = ctypes.c_void_p


def build(verbose: bool = False) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-o", _LIB_PATH,
           os.path.join(_HERE, "synth.c"), "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.synth_philox4x32_10.argtypes = [VP, VP, VP]
        L.synth_normal_f32.argtypes = [U64, U32, U64, U64, F32, VP, I32]
        L.synth_normal_bf16.argtypes = [U64, U32, U64, U64, F32, VP, I32]
        L.synth_intgrid_f32.argtypes = [U64, U32, U64, U64, I32, I32, VP, I32]
        L.synth_intgrid_bf16.argtypes = [U64, U32, U64, U64, I32, I32, VP, I32]
        L.synth_u32.argtypes = [U64, U32, U64, U64, VP]
        L.synth_mxfp4.argtypes = [U64, U32, U64, U64, U64, F32, VP, VP, I32]
        L.synth_mxfp4_intgrid.argtypes = [U64, U32, U64, U64, U64, I32, I32, VP, VP, I32]
        L.synth_fp8_rows.argtypes = [U64, U32, U64, U64, U64, F32, VP, VP, I32]
        L.synth_fp8_rows_intgrid.argtypes = [U64, U32, U64, U64, U64, I32, I32, VP, VP, I32]
        for f in ("synth_philox4x32_10", "synth_normal_f32", "synth_normal_bf16", "synth_intgrid_f32",
                  "synth_intgrid_bf16", "synth_u32", "synth_mxfp4", "synth_mxfp4_intgrid", "synth_fp8_rows",
                  "synth_fp8_rows_intgrid"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def threads() -> int:
    """Worker threads for host generation: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    o = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def normal(seed, tid, shape, sigma=1.0, dtype="f32", offset=0) -> np.ndarray:
    """sigma * N(0,1); dtype 'f32' (float32) or 'bf16' (uint16 holding bf16 bits)."""
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        lib().synth_normal_f32(seed, tid, offset, n, sigma, _ptr(out), threads())
    else:
        out = np.empty(shape, dtype=np.uint16)
        lib().synth_normal_bf16(seed, tid, offset, n, sigma, _ptr(out), threads())
    return out


def intgrid(seed, tid, shape, lo, hi, dtype="f32", offset=0) -> np.ndarray:
    """Uniform integers in [lo, hi], as float32 or bf16 bits."""
    n = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        lib().synth_intgrid_f32(seed, tid, offset, n, lo, hi, _ptr(out), threads())
    else:
        out = np.empty(shape, dtype=np.uint16)
        lib().synth_intgrid_bf16(seed, tid, offset, n, lo, hi, _ptr(out), threads())
    return out


def u32(seed, tid, n, offset=0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().synth_u32(seed, tid, offset, n, _ptr(out))
    return out


def mxfp4(seed, tid, G, R, K, sigma, grid=None):
    """[G, R, K] weight drawn N(0, sigma^2) (or integers in grid=(lo, hi)), quantised to MXFP4.

    Returns (codes uint8 [G, R, K/2], scales uint8 [G, R, K/32]).
    """
    assert K % 32 == 0
    codes = np.empty((G, R, K // 2), dtype=np.uint8)
    scales = np.empty((G, R, K // 32), dtype=np.uint8)
    if grid is None:
        lib().synth_mxfp4(seed, tid, 0, G * R, K, sigma, _ptr(codes), _ptr(scales), threads())
    else:
        lib().synth_mxfp4_intgrid(seed, tid, 0, G * R, K, grid[0], grid[1], _ptr(codes), _ptr(scales),
                                  threads())
    return codes, scales


def fp8_rows(seed, tid, rows, K, sigma, grid=None, row0=0):
    """[rows, K] drawn N(0, sigma^2) (or integers in grid=(lo, hi), scale 1), encoded as FP8 e4m3
    with one power-of-two fp32 scale per 128 along K (the OCP MX v1.0 scale rule, E4M3
    elements).  Returns (codes uint8 [rows, K], scales float32 [rows, K/128])."""
    assert K % 128 == 0
    codes = np.empty((rows, K), dtype=np.uint8)
    scales = np.empty((rows, K // 128), dtype=np.float32)
    if grid is None:
        lib().synth_fp8_rows(seed, tid, row0, rows, K, sigma, _ptr(codes), _ptr(scales), threads())
    else:
        lib().synth_fp8_rows_intgrid(seed, tid, row0, rows, K, grid[0], grid[1], _ptr(codes), _ptr(scales),
                                     threads())
    return codes, scales


# ---------------------------------------------------------------------------
# workload definitions
# ---------------------------------------------------------------------------

MODE_F32, MODE_BF16, MODE_FP8, MODE_FP8X8 = "f32", "bf16", "fp8_mxfp4", "fp8_fp8"
TID_X, TID_WR, TID_BIASPERM, TID_W1, TID_W2 = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    mode: str
    T: int
    d: int
    E: int
    k: int
    F: int
    S: int
    gating: str           # "softmax" | "sigmoid"
    zipf_alpha: float = 0.0
    zipf_s: float = 1.1
    t_values: tuple = field(default=())

    @property
    def G(self) -> int:
        return self.E + self.S

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1001, MODE_F32, 64, 128, 8, 2, 256, 0, "softmax"),
    "mixtral_bf16": Workload("mixtral_bf16", 1002, MODE_BF16, 4096, 4096, 8, 2, 14336, 0, "softmax"),
    "dsv3_bf16": Workload("dsv3_bf16", 1003, MODE_BF16, 8192, 7168, 256, 8, 2048, 1, "sigmoid",
                          zipf_alpha=0.25),
    "dsv3_fp8fp4": Workload("dsv3_fp8fp4", 1004, MODE_FP8, 8192, 7168, 256, 8, 2048, 1, "softmax",
                            t_values=(512, 8192, 32768)),
    # the DeepSeek-V3 shape with FP8 e4m3 weights (1x128 power-of-two scales) as well
    "dsv3_fp8fp8": Workload("dsv3_fp8fp8", 1006, MODE_FP8X8, 8192, 7168, 256, 8, 2048, 1, "softmax",
                            t_values=(8192,)),
    # the same layer (same seed, so the same tensors) at decode batch sizes
    "decode_fp8fp4": Workload("decode_fp8fp4", 1004, MODE_FP8, 1, 7168, 256, 8, 2048, 1, "softmax",
                              t_values=(1, 64)),
    # the same layer with the DeepSeek-V3-shaped router: sigmoid scores and Zipf-skewed bias
    "dsv3_fp8fp4_zipf": Workload("dsv3_fp8fp4_zipf", 1004, MODE_FP8, 8192, 7168, 256, 8, 2048, 1, "sigmoid",
                                 zipf_alpha=0.25, t_values=(8192,)),
}


def zipf_bias(w: Workload) -> np.ndarray | None:
    """Per-expert selection bias b_e = alpha * r_e^(-s), ranks r_e a seeded permutation of 1..E."""
    if w.zipf_alpha == 0.0:
        return None
    keys = u32(w.seed, TID_BIASPERM, w.E)
    order = np.argsort(keys, kind="stable")
    rank = np.empty(w.E, dtype=np.int64)
    rank[order] = np.arange(1, w.E + 1)
    return (w.zipf_alpha * rank.astype(np.float64) ** (-w.zipf_s)).astype(np.float32)


def make_inputs(w: Workload, grid: bool = False, zero_gate: bool = False) -> dict:
    """All layer inputs as numpy arrays.

    f32 mode:  x, w_router, w1 [G,2F,d], w2 [G,d,F] as float32.
    bf16 mode: the same as uint16 bf16 bits.
    fp8 mode:  x, w_router bf16 bits; w1/w2 MXFP4 codes with w1_scale/w2_scale e8m0.
    fp8_fp8:   x, w_router bf16 bits; w1/w2 e4m3 codes with fp32 scales per 1x128.
    grid=True draws small integers instead of normals, so every product sum is exact.
    """
    s, T, d, E, F, G = w.seed, w.T, w.d, w.E, w.F, w.G
    act = "f32" if w.mode == MODE_F32 else "bf16"
    out = {"workload": w}
    if grid:
        out["x"] = intgrid(s, TID_X, (T, d), -2, 2, act)
        out["w_router"] = intgrid(s, TID_WR, (E, d), -2, 2, act)
    else:
        out["x"] = normal(s, TID_X, (T, d), 1.0, act)
        out["w_router"] = normal(s, TID_WR, (E, d), 1.0 / math.sqrt(d), act)
    out["bias"] = zipf_bias(w)
    if w.mode == MODE_FP8:
        if grid:
            out["w1"], out["w1_scale"] = mxfp4(s, TID_W1, G, 2 * F, d, 0.0, grid=(-2, 2))
            out["w2"], out["w2_scale"] = mxfp4(s, TID_W2, G, d, F, 0.0, grid=(-2, 2))
        else:
            out["w1"], out["w1_scale"] = mxfp4(s, TID_W1, G, 2 * F, d, 1.0 / math.sqrt(d))
            out["w2"], out["w2_scale"] = mxfp4(s, TID_W2, G, d, F, 1.0 / math.sqrt(F))
    elif w.mode == MODE_FP8X8:
        g = (-2, 2) if grid else None
        c1, s1 = fp8_rows(s, TID_W1, G * 2 * F, d, 1.0 / math.sqrt(d), grid=g)
        c2, s2 = fp8_rows(s, TID_W2, G * d, F, 1.0 / math.sqrt(F), grid=g)
        out["w1"], out["w1_scale"] = c1.reshape(G, 2 * F, d), s1.reshape(G, 2 * F, d // 128)
        out["w2"], out["w2_scale"] = c2.reshape(G, d, F), s2.reshape(G, d, F // 128)
    else:
        if grid:
            out["w1"] = intgrid(s, TID_W1, (G, 2 * F, d), -2, 2, act)
            out["w2"] = intgrid(s, TID_W2, (G, d, F), -2, 2, act)
        else:
            out["w1"] = normal(s, TID_W1, (G, 2 * F, d), 1.0 / math.sqrt(d), act)
            out["w2"] = normal(s, TID_W2, (G, d, F), 1.0 / math.sqrt(F), act)
        out["w1_scale"] = out["w2_scale"] = None
    if zero_gate:
        out["w1"][:, :F, :] = 0
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) -> float32, exact."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)
