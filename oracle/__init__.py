"""CPU oracle for the MoE-layer forward (ctypes over ``liboracle.so``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.  It shares no code with
the GPU path; both only receive the arrays the ``synth`` generators write.

Every function here marshals numpy arrays into the C oracle (``moe_oracle.c``),
which holds the arithmetic and cites the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

MODES = {"f32": 0, "bf16": 1, "fp8_mxfp4": 2, "fp8_fp8": 3}
GATINGS = {"softmax": 0, "sigmoid": 1}
STATUS = {0: "ok", 1: "expert index out of range", 2: "duplicate expert for a token",
          3: "non-finite selection key", 4: "bad shape"}


class OracleError(RuntimeError):
    pass


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "d", "E", "k", "F", "S", "gating", "mode")]


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc; no fast-math and no FMA contraction."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-ffp-contract=off", "-fno-fast-math",
           "-o", _LIB_PATH, os.path.join(_HERE, "moe_oracle.c"), "-lm", "-lpthread"]
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
        VP, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        CP = ctypes.POINTER(_Cfg)
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_block_exponent.argtypes = [ctypes.c_float]
        L.oracle_e4m3_block_exponent.restype = I32
        L.oracle_quant_e4m3_b128.argtypes = [VP, I64, VP, VP]
        L.oracle_quant_e4m3_b128.restype = None
        L.oracle_route.argtypes = [CP, VP, VP, VP, VP, VP, VP, VP, I32]
        L.oracle_route.restype = I32
        L.oracle_topk_gates_from.argtypes = [CP, VP, VP, VP, VP]
        L.oracle_topk_gates_from.restype = I32
        L.oracle_dispatch.argtypes = [CP, VP, VP, VP, VP, VP]
        L.oracle_dispatch.restype = I32
        L.oracle_layer.argtypes = [CP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, I64, VP, VP, VP, I32]
        L.oracle_layer.restype = I32
        L.oracle_expert_rows.argtypes = [CP, VP, VP, VP, VP, I32, VP, I64, VP, VP]
        L.oracle_expert_rows.restype = None
        L.oracle_down_rows.argtypes = [CP, VP, VP, I32, VP, I64, VP]
        L.oracle_down_rows.restype = None
        L.oracle_layer_dropping.argtypes = [CP, VP, VP, VP, VP, VP, VP, VP, VP, VP, I64, VP, I32]
        L.oracle_layer_dropping.restype = I32
        L.oracle_dispatch_capacity.argtypes = [CP, VP, I32, VP, VP, VP, VP, VP]
        L.oracle_dispatch_capacity.restype = I32
        L.oracle_bias_update.argtypes = [I32, VP, VP, ctypes.c_float]
        L.oracle_bias_update.restype = None
        L.oracle_dequant_e4m3_rows.argtypes = [VP, VP, I64, I64, VP]
        L.oracle_dequant_e4m3_rows.restype = None
        L.oracle_gemm_fp8_mxfp4.argtypes = [I64, I64, I64, VP, VP, VP, VP, VP]
        L.oracle_gemm_fp8_mxfp4.restype = None
        L.oracle_keys_from.argtypes = [CP, VP, VP, VP]
        L.oracle_keys_from.restype = None
        L.oracle_input_row.argtypes = [CP, VP, I64, VP]
        L.oracle_input_row.restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "arrays must be C-contiguous numpy"
    return a.ctypes.data


def _cfg(w, T=None) -> _Cfg:
    return _Cfg(T if T is not None else w.T, w.d, w.E, w.k, w.F, w.S, GATINGS[w.gating], MODES[w.mode])


def _check(st):
    if st != 0:
        raise OracleError(STATUS.get(st, f"status {st}"))


# ---- number formats ---------------------------------------------------------

def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(code)


def e2m1_decode(code: int) -> float:
    return lib().oracle_e2m1_decode(code)


def e8m0_decode(code: int) -> float:
    return lib().oracle_e8m0_decode(code)


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(v)


def e4m3_block_exponent(amax: float) -> int:
    return lib().oracle_e4m3_block_exponent(amax)


def quant_e4m3_b128(v: np.ndarray):
    """Rows of fp32 values (last dim a multiple of 128) -> (e4m3 codes, fp32 power-of-two scales)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    n = v.size
    assert v.shape[-1] % 128 == 0
    codes = np.empty(v.shape, dtype=np.uint8)
    scales = np.empty(v.shape[:-1] + (v.shape[-1] // 128,), dtype=np.float32)
    lib().oracle_quant_e4m3_b128(_p(v), n, _p(codes), _p(scales))
    return codes, scales


# ---- routing ------------------------------------------------------------------

def route(inp: dict, nthreads: int = 0, T: int | None = None):
    """S1-S4 over all tokens -> dict(idx [T,k] int32, gates [T,k] f32, logits, keys [T,E] f32)."""
    w = inp["workload"]
    T = w.T if T is None else T
    c = _cfg(w, T)
    idx = np.empty((T, w.k), dtype=np.int32)
    gates = np.empty((T, w.k), dtype=np.float32)
    logits = np.empty((T, w.E), dtype=np.float32)
    keys = np.empty((T, w.E), dtype=np.float32)
    _check(lib().oracle_route(ctypes.byref(c), _p(inp["x"]), _p(inp["w_router"]), _p(inp["bias"]),
                              _p(idx), _p(gates), _p(logits), _p(keys), nthreads))
    return {"idx": idx, "gates": gates, "logits": logits, "keys": keys}


def topk_gates_from(w, logits: np.ndarray, keys: np.ndarray):
    """Top-k + gates from given logits/keys [T,E] (fp32)."""
    T = logits.shape[0]
    c = _cfg(w, T)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    keys = np.ascontiguousarray(keys, dtype=np.float32)
    idx = np.empty((T, w.k), dtype=np.int32)
    gates = np.empty((T, w.k), dtype=np.float32)
    _check(lib().oracle_topk_gates_from(ctypes.byref(c), _p(logits), _p(keys), _p(idx), _p(gates)))
    return idx, gates


def keys_from_logits(w, logits: np.ndarray, bias=None) -> np.ndarray:
    """Selection keys [T,E] from given fp32 logits (softmax: l + b; sigmoid: sigmoid(l) + b)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    c = _cfg(w, logits.shape[0])
    keys = np.empty_like(logits)
    lib().oracle_keys_from(ctypes.byref(c), _p(logits), _p(bias), _p(keys))
    return keys


def dispatch(w, idx: np.ndarray):
    """S5-S6 -> dict(counts [G], offsets [G+1], slot_to_row [T*k], row_to_slot [T*k])."""
    T = idx.shape[0]
    c = _cfg(w, T)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    G = w.E + w.S
    counts = np.empty(G, dtype=np.int32)
    offsets = np.empty(G + 1, dtype=np.int32)
    s2r = np.empty(T * w.k, dtype=np.int32)
    r2s = np.empty(T * w.k, dtype=np.int32)
    _check(lib().oracle_dispatch(ctypes.byref(c), _p(idx), _p(counts), _p(offsets), _p(s2r), _p(r2s)))
    return {"counts": counts, "offsets": offsets, "slot_to_row": s2r, "row_to_slot": r2s}


def dispatch_capacity(w, idx: np.ndarray, capacity: int):
    """The capacity variant of S5-S6: at most `capacity` slots per routed expert, the first
    ones in slot order kept -> dict(counts [G] (kept), dropped [E], offsets [G+1],
    slot_to_row [T*k] (-1 when dropped), row_to_slot [T*k])."""
    T = idx.shape[0]
    c = _cfg(w, T)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    G = w.E + w.S
    counts = np.empty(G, dtype=np.int32)
    dropped = np.empty(w.E, dtype=np.int32)
    offsets = np.empty(G + 1, dtype=np.int32)
    s2r = np.empty(T * w.k, dtype=np.int32)
    r2s = np.empty(T * w.k, dtype=np.int32)
    _check(lib().oracle_dispatch_capacity(ctypes.byref(c), _p(idx), int(capacity), _p(counts), _p(dropped),
                                          _p(offsets), _p(s2r), _p(r2s)))
    return {"counts": counts, "dropped": dropped, "offsets": offsets, "slot_to_row": s2r, "row_to_slot": r2s}


def bias_update(counts: np.ndarray, bias: np.ndarray, gamma: float) -> np.ndarray:
    """One aux-loss-free bias update from routed per-expert counts [E] -> new bias [E] (fp32)."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    out = np.ascontiguousarray(bias, dtype=np.float32).copy()
    lib().oracle_bias_update(counts.size, _p(counts), _p(out), float(gamma))
    return out


# ---- experts and the layer -------------------------------------------------------

def input_rows(inp: dict, tokens) -> np.ndarray:
    """Expert input rows in fp64: x, or its e4m3 1x128 dequantisation in FP8 mode."""
    w = inp["workload"]
    c = _cfg(w)
    out = np.empty((len(tokens), w.d), dtype=np.float64)
    for n, t in enumerate(tokens):
        lib().oracle_input_row(ctypes.byref(c), _p(inp["x"]), int(t), out[n].ctypes.data)
    return out


def expert_rows(inp: dict, g: int, xin: np.ndarray, want_h: bool = False):
    """Expert g applied to fp64 input rows [n, d] -> out [n, d] (and h [n, F] before FP8 rounding)."""
    w = inp["workload"]
    c = _cfg(w)
    xin = np.ascontiguousarray(xin, dtype=np.float64)
    n = xin.shape[0]
    out = np.empty((n, w.d), dtype=np.float64)
    h = np.empty((n, w.F), dtype=np.float64) if want_h else None
    lib().oracle_expert_rows(ctypes.byref(c), _p(inp["w1"]), _p(inp["w1_scale"]), _p(inp["w2"]),
                             _p(inp["w2_scale"]), int(g), _p(xin), n, _p(out), _p(h))
    return (out, h) if want_h else out


def down_rows(inp: dict, g: int, hhat: np.ndarray) -> np.ndarray:
    """linear2 of expert g on given fp64 rows hhat [n, F] (in FP8 mode: dequantised e4m3 h)
    -> [n, d]."""
    w = inp["workload"]
    c = _cfg(w)
    hhat = np.ascontiguousarray(hhat, dtype=np.float64)
    n = hhat.shape[0]
    out = np.empty((n, w.d), dtype=np.float64)
    lib().oracle_down_rows(ctypes.byref(c), _p(inp["w2"]), _p(inp["w2_scale"]), int(g), _p(hhat), n, _p(out))
    return out


def dequant_e4m3_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """e4m3 codes [n, K] and fp32 scales [n, K/128] -> fp64 values [n, K]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    n, K = codes.shape
    out = np.empty((n, K), dtype=np.float64)
    lib().oracle_dequant_e4m3_rows(_p(codes), _p(scales), n, K, _p(out))
    return out


def gemm_fp8_mxfp4(a, a_scale, b, b_scale, rows=None) -> np.ndarray:
    """Dense FP8 x MXFP4 GEMM: A codes [M, K] + scales [M, K/128], B MXFP4 [N, K/2] + e8m0
    [N, K/32] -> C [M, N] fp64 (for the listed rows of A only, when given)."""
    a = np.ascontiguousarray(a if rows is None else a[rows], dtype=np.uint8)
    a_scale = np.ascontiguousarray(a_scale if rows is None else a_scale[rows], dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    b_scale = np.ascontiguousarray(b_scale, dtype=np.uint8)
    M, K = a.shape
    N = b.shape[0]
    c = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm_fp8_mxfp4(M, N, K, _p(a), _p(a_scale), _p(b), _p(b_scale), _p(c))
    return c


def layer_dropping(inp: dict, idx, gates, keep, tokens=None, nthreads: int = 0):
    """y [ntok, d] fp64 under the capacity variant: the given routing, minus the dropped slots
    (keep [T, k] false); their gates are not renormalised."""
    w = inp["workload"]
    T = inp["x"].shape[0]
    c = _cfg(w, T)
    tokens = np.arange(T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = tokens.shape[0]
    y = np.empty((n, w.d), dtype=np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    gates = np.ascontiguousarray(gates, dtype=np.float32)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    _check(lib().oracle_layer_dropping(ctypes.byref(c), _p(inp["x"]), _p(inp["w1"]), _p(inp["w1_scale"]),
                                       _p(inp["w2"]), _p(inp["w2_scale"]), _p(idx), _p(gates), _p(keep),
                                       _p(tokens), n, _p(y), nthreads))
    return y


def layer(inp: dict, tokens=None, idx=None, gates=None, nthreads: int = 0):
    """y [ntok, d] fp64 for the listed tokens (all by default).

    With idx/gates ([T,k], e.g. another implementation's routing) the oracle uses
    that routing; otherwise it routes itself.  Returns (y, idx_used, gates_used).
    """
    w = inp["workload"]
    T = inp["x"].shape[0]
    c = _cfg(w, T)
    tokens = np.arange(T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = tokens.shape[0]
    y = np.empty((n, w.d), dtype=np.float64)
    iu = np.empty((n, w.k), dtype=np.int32)
    gu = np.empty((n, w.k), dtype=np.float32)
    if idx is not None:
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        gates = np.ascontiguousarray(gates, dtype=np.float32)
    _check(lib().oracle_layer(ctypes.byref(c), _p(inp["x"]), _p(inp["w_router"]), _p(inp["bias"]),
                              _p(inp["w1"]), _p(inp["w1_scale"]), _p(inp["w2"]), _p(inp["w2_scale"]),
                              _p(idx), _p(gates), _p(tokens), n, _p(y), _p(iu), _p(gu), nthreads))
    return y, iu, gu
