"""ctypes front end of the CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg import this module. It never touches the HIP
library, and the HIP library never calls it.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FMT_MXFP4, FMT_NVFP4, FMT_NF3 = 1, 2, 3
# activation forms (orc_act): SwiGLU (limit clamps, OAI alpha / beta), SiTU, ReLU^2 without the gate multiply
ACT_SWIGLU, ACT_SITU, ACT_RELU2_NO_MUL = 0, 1, 2


class _Tier(C.Structure):
    _fields_ = [("fmt", C.c_int), ("E", C.c_int), ("emap", C.c_void_p),
                ("w13", C.c_void_p), ("s13", C.c_void_p), ("g13", C.c_void_p),
                ("w2", C.c_void_p), ("s2", C.c_void_p), ("g2", C.c_void_p)]


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "moe_oracle.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.orc_e2m1.restype = C.c_double
        L.orc_e2m1.argtypes = [C.c_uint]
        L.orc_e8m0.restype = C.c_double
        L.orc_e8m0.argtypes = [C.c_uint]
        L.orc_e4m3.restype = C.c_double
        L.orc_e4m3.argtypes = [C.c_uint]
        L.orc_nf3.restype = C.c_double
        L.orc_nf3.argtypes = [C.c_uint]
        L.orc_e4m3_encode.restype = C.c_uint
        L.orc_e4m3_encode.argtypes = [C.c_double]
        L.orc_bf16_to_double.restype = C.c_double
        L.orc_bf16_to_double.argtypes = [C.c_uint16]
        L.orc_bf16_from_double.restype = C.c_uint16
        L.orc_bf16_from_double.argtypes = [C.c_double]
        for n in ("orc_mxfp8_quantize_f32", "orc_mxfp8_quantize_bf16"):
            getattr(L, n).restype = C.c_int
            getattr(L, n).argtypes = [C.c_void_p, C.c_long, C.c_long, C.c_void_p, C.c_void_p]
        L.orc_dequant.restype = C.c_int
        L.orc_dequant.argtypes = [C.c_int, C.c_void_p, C.c_void_p, C.c_double, C.c_long, C.c_long, C.c_void_p]
        L.orc_route.restype = C.c_long
        L.orc_route.argtypes = [C.c_void_p, C.c_long, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.orc_moe.restype = C.c_int
        L.orc_moe.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_double, C.c_int, C.c_int, C.c_void_p,
                              C.c_void_p, C.c_void_p, C.c_void_p, C.c_long, C.c_void_p, C.c_long,
                              C.c_void_p, C.c_void_p]
        L.orc_moe_ex.restype = C.c_int
        L.orc_moe_ex.argtypes = L.orc_moe.argtypes + [C.c_int, C.c_double, C.c_double]
        L.orc_moe_act.restype = C.c_int
        L.orc_moe_act.argtypes = L.orc_moe_ex.argtypes + [C.c_int]
        L.orc_act.restype = C.c_double
        L.orc_act.argtypes = [C.c_int, C.c_double, C.c_double, C.c_double, C.c_double, C.c_double]
        L.orc_ep_remap.restype = C.c_int
        L.orc_ep_remap.argtypes = [C.c_void_p, C.c_void_p, C.c_long, C.c_int, C.c_long, C.c_long,
                                   C.c_void_p, C.c_void_p]
        L.orc_num_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ scalars
def e2m1(code: int) -> float:
    return lib().orc_e2m1(code)


def e8m0(b: int) -> float:
    return lib().orc_e8m0(b)


def e4m3(b: int) -> float:
    return lib().orc_e4m3(b)


def nf3(code: int) -> float:
    return lib().orc_nf3(code)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def bf16_to_float(h: int) -> float:
    return lib().orc_bf16_to_double(h)


def bf16_from_float(d: float) -> int:
    return lib().orc_bf16_from_double(float(d))


def act(kind: int, gate: float, up: float, limit=None, alpha: float = 1.0, beta: float = 0.0) -> float:
    """The activation the layer applies to one (gate, up) pair (orc_act; ReLU^2 reads up only)."""
    lim = math.nan if limit is None else float(limit)
    return lib().orc_act(int(kind), float(gate), float(up), lim, float(alpha), float(beta))


def ep_remap(ids: np.ndarray, w: np.ndarray, offset: int, num_local: int):
    """Expert-parallel id remap of [T, k] ids / weights (sglang moe_b12x_next.py, ep_remap_reference):
    returns (local ids int32 [T, k], weights float32 [T, k])."""
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    T, k = ids.shape
    oi = np.empty((T, k), np.int32)
    ow = np.empty((T, k), np.float32)
    if lib().orc_ep_remap(_p(ids), _p(w), T, k, int(offset), int(num_local), _p(oi), _p(ow)) != 0:
        raise ValueError("bad remap arguments")
    return oi, ow


# ------------------------------------------------------------------ arrays
def mxfp8_quantize_f32(v: np.ndarray):
    """[rows, cols] fp32 -> (codes u8 [rows, cols], scales u8 [rows, cols/32])."""
    v = _c(v, np.float32)
    rows, cols = v.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 32), np.uint8)
    if lib().orc_mxfp8_quantize_f32(_p(v), rows, cols, _p(q), _p(s)) != 0:
        raise ValueError("cols must be a multiple of 32")
    return q, s


def mxfp8_quantize_bf16(x: np.ndarray):
    """[rows, cols] bf16 bit patterns (uint16) -> (codes, scales)."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 32), np.uint8)
    if lib().orc_mxfp8_quantize_bf16(_p(x), rows, cols, _p(q), _p(s)) != 0:
        raise ValueError("cols must be a multiple of 32")
    return q, s


def dequant(fmt: int, w: np.ndarray, s: np.ndarray, cols: int, g: float = 1.0) -> np.ndarray:
    """One expert's checkpoint matrix [rows, packed] -> float64 [rows, cols]."""
    w = _c(w, np.uint8)
    s = _c(s, np.uint8)
    rows = w.shape[0]
    out = np.empty((rows, cols), np.float64)
    if lib().orc_dequant(fmt, _p(w), _p(s), float(g), rows, cols, _p(out)) != 0:
        raise ValueError("bad format or shape")
    return out


class _TierArgs:
    """Keeps the numpy buffers of the tier structs alive for one call."""

    def __init__(self, tiers):
        self.keep = []
        arr = (_Tier * len(tiers))()
        for i, t in enumerate(tiers):
            w = t.weights
            fields = {}
            for key, dt in (("w13", np.uint8), ("s13", np.uint8), ("w2", np.uint8), ("s2", np.uint8),
                            ("g13", np.float32), ("g2", np.float32)):
                a = _c(w.get(key), dt)
                self.keep.append(a)
                fields[key] = _p(a)
            em = _c(t.emap, np.int32)
            self.keep.append(em)
            arr[i] = _Tier(t.fmt, t.E, _p(em), fields["w13"], fields["s13"], fields["g13"],
                           fields["w2"], fields["s2"], fields["g2"])
        self.arr = arr


def route(ids: np.ndarray, E_global: int, tiers):
    """Route planner definition. Returns (cnt [U], off [U+1], perm [R_valid], inv [T*k])."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    U = sum(t.E for t in tiers)
    cnt = np.empty(U, np.int32)
    off = np.empty(U + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    ta = _TierArgs(tiers)
    n = lib().orc_route(_p(ids), T, k, E_global, len(tiers), C.addressof(ta.arr), _p(cnt), _p(off),
                        _p(perm), _p(inv))
    if n < 0:
        raise ValueError("bad routing arguments")
    return cnt, off, perm[:n].copy(), inv


def moe(E_global: int, K: int, N: int, topk: int, limit, tiers, x: np.ndarray, ids: np.ndarray,
        wts: np.ndarray, rows=None, gate_up: bool = False, weight_on_input: bool = False,
        alpha: float = 1.0, beta: float = 0.0, act_kind: int = ACT_SWIGLU):
    """The layer for the listed token rows (all rows when None).  weight_on_input:
    each slot's router weight scales that slot's copy of the token before GEMM1 and
    its result enters the sum with weight 1 (vLLM "fused_moe/b12x" page,
    apply_router_weight_on_input; 16-bit activation formats only).  alpha, beta:
    the activation gate * sigmoid(alpha gate) * (up + beta) after the clamps
    (swigluoai's parameters on the same page, _swiglu_params; 1, 0 is SwiGLU;
    other values 16-bit activation formats only).  act_kind: ACT_SITU or
    ACT_RELU2_NO_MUL instead of the SwiGLU (no limit, alpha or beta; ReLU^2 reads a
    w13 of N rows and runs with 16-bit activation formats only).

    Returns (acc float64 [n, K], out bf16-bits uint16 [n, K])."""
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32)
    wts = _c(wts, np.float32)
    T = x.shape[0]
    rows_a = None if rows is None else _c(np.asarray(rows), np.int32)
    n = T if rows_a is None else rows_a.shape[0]
    acc = np.empty((n, K), np.float64)
    out = np.empty((n, K), np.uint16)
    ta = _TierArgs(tiers)
    lim = math.nan if limit is None else float(limit)
    rc = lib().orc_moe_act(E_global, K, N, topk, lim, int(gate_up), len(tiers), C.addressof(ta.arr), _p(x),
                           _p(ids), _p(wts), T, _p(rows_a), n, _p(acc), _p(out), int(bool(weight_on_input)),
                           float(alpha), float(beta), int(act_kind))
    if rc != 0:
        raise ValueError("bad layer arguments")
    return acc, out


def moe_problem(prob, rows=None, gate_up: bool = False, weight_on_input: bool = False, alpha: float = 1.0,
                beta: float = 0.0, act_kind: int = ACT_SWIGLU):
    """The layer for a block_scaled_fp4_histogram_amd.inputs.Problem."""
    c = prob.cfg
    limit = c.limit if act_kind == ACT_SWIGLU else None
    return moe(c.E, c.K, c.N, c.topk, limit, prob.tiers, prob.x, prob.ids, prob.wts, rows, gate_up,
               weight_on_input, alpha, beta, act_kind)


def num_threads() -> int:
    return lib().orc_num_threads()
