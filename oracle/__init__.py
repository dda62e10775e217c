"""CPU oracle of the MoE layer forward pass — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``liboracle.so`` (built from ``oracle.cpp`` with
g++ -O2 -ffp-contract=off -fopenmp) with numpy arrays; it shares no code with
the HIP library.  The arithmetic and the page citations are in ``oracle.cpp``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

ACT = {"f32": 0, "bf16": 1}
WDT = {"f32": 0, "bf16": 1, "mxfp4": 2}
ROUTE = {"softmax": 0, "sigmoid": 1, "hash": 2}
GLU = {"swiglu": 0, "clamp": 1, "situ": 2}

_lib = None


class _Experts(ctypes.Structure):
    _fields_ = [("wdtype", ctypes.c_int),
                ("gate", ctypes.POINTER(ctypes.c_void_p)),
                ("up", ctypes.POINTER(ctypes.c_void_p)),
                ("down", ctypes.POINTER(ctypes.c_void_p)),
                ("gate_scale", ctypes.POINTER(ctypes.c_void_p)),
                ("up_scale", ctypes.POINTER(ctypes.c_void_p)),
                ("down_scale", ctypes.POINTER(ctypes.c_void_p))]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.orc_exp.argtypes, L.orc_exp.restype = [f32], f32
        L.orc_glu_value.argtypes = [ctypes.c_double, ctypes.c_double, i32]
        L.orc_glu_value.restype = ctypes.c_double
        L.orc_sigmoid.argtypes, L.orc_sigmoid.restype = [f32], f32
        L.orc_bf16_from_f64.argtypes, L.orc_bf16_from_f64.restype = [ctypes.c_double], ctypes.c_uint16
        L.orc_bf16_from_f32.argtypes, L.orc_bf16_from_f32.restype = [f32], ctypes.c_uint16
        L.orc_mxfp4_value.argtypes = [ctypes.c_uint8, ctypes.c_uint8]
        L.orc_mxfp4_value.restype = ctypes.c_double
        L.orc_fmix32.argtypes, L.orc_fmix32.restype = [ctypes.c_uint32], ctypes.c_uint32
        L.orc_exp_array.argtypes = [vp, vp, i64]
        L.orc_sigmoid_array.argtypes = [vp, vp, i64]
        L.orc_bf16_from_f64_array.argtypes = [vp, vp, i64]
        L.orc_router_logits.argtypes = [vp, i32, vp, i64, i32, i32, vp]
        L.orc_route.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp, vp, vp]
        L.orc_route.restype = i32
        L.orc_permute.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
        L.orc_permute.restype = i32
        L.orc_expert_ffn.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                     i32]
        L.orc_combine.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, vp]
        L.orc_residual_rmsnorm.argtypes = [vp, vp, vp, ctypes.c_double, i64, i32, i32, vp, vp]
        L.orc_e4m3_value.argtypes, L.orc_e4m3_value.restype = [ctypes.c_uint8], ctypes.c_double
        L.orc_e4m3_round.argtypes, L.orc_e4m3_round.restype = [ctypes.c_double], ctypes.c_uint8
        L.orc_mx_e4m3_quantize.argtypes = [vp, i64, i64, vp, vp]
        L.orc_expert_ffn_w4a8.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        L.orc_layer_forward.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(_Experts), vp, vp, vp,
                                        i64, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, i32]
        L.orc_layer_forward.restype = i32
        L.orc_num_threads.restype = i32
        L.orc_set_num_threads.argtypes = [i32]
        L.orc_set_num_threads.restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], type(a)
    return a.ctypes.data


def act_name(arr: np.ndarray) -> str:
    return "f32" if arr.dtype == np.float32 else "bf16"


def exp(x: float) -> float:
    return lib().orc_exp(x)


def sigmoid(x: float) -> float:
    return lib().orc_sigmoid(x)


def glu_value(g: float, u: float, glu: str = "swiglu") -> float:
    """Gated activation of one (gate, up) pair in double (see glu_value in oracle.cpp)."""
    return lib().orc_glu_value(g, u, GLU[glu])


def exp_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().orc_exp_array(_p(x), _p(out), x.size)
    return out


def sigmoid_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().orc_sigmoid_array(_p(x), _p(out), x.size)
    return out


def bf16_from_f64_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_from_f64_array(_p(x), _p(out), x.size)
    return out


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    T, D = x.shape
    E = w_router.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(_p(x), ACT[act_name(x)], _p(w_router), T, D, E, _p(out))
    return out


def route(logits, bias, token_ids, T, E, k, mode, want_keys=False):
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    keys = np.empty((T, E), dtype=np.float32) if want_keys else None
    rc = lib().orc_route(_p(logits), _p(bias), _p(token_ids), T, E, k, ROUTE[mode],
                         _p(idx), _p(w), _p(keys))
    if rc != 0:
        raise ValueError(f"orc_route rc={rc}")
    return (idx, w, keys) if want_keys else (idx, w)


def permute(topk_idx: np.ndarray, E: int):
    T, k = topk_idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    row_token = np.empty(T * k, dtype=np.int32)
    pair_row = np.empty(T * k, dtype=np.int32)
    rc = lib().orc_permute(_p(np.ascontiguousarray(topk_idx, dtype=np.int32)), T, k, E,
                           _p(counts), _p(offsets), _p(row_token), _p(pair_row))
    if rc != 0:
        raise ValueError(f"orc_permute rc={rc}")
    return counts, offsets, row_token, pair_row


def expert_ffn(x_rows: np.ndarray, gate, up, down, wdtype: str, want_h=False, glu="swiglu"):
    """One expert over M rows.  For mxfp4 each weight is a (codes, scales) pair.
    glu: "swiglu", "clamp" or "situ" (the gated activation)."""
    M, D = x_rows.shape
    act = act_name(x_rows)
    if wdtype == "mxfp4":
        (g, gs), (u, us), (d, ds) = gate, up, down
        I = g.shape[0]
    else:
        g, u, d = gate, up, down
        gs = us = ds = None
        I = g.shape[0]
    out = np.empty((M, D), dtype=x_rows.dtype)
    h = np.empty((M, I), dtype=x_rows.dtype) if want_h else None
    lib().orc_expert_ffn(_p(x_rows), ACT[act], M, D, I, WDT[wdtype], _p(g), _p(u), _p(d),
                         _p(gs), _p(us), _p(ds), _p(out), _p(h), GLU[glu])
    return (out, h) if want_h else out


def e4m3_value(code: int) -> float:
    """OCP FP8 E4M3 (no infinities) value of a code byte."""
    return lib().orc_e4m3_value(code)


def e4m3_round(v: float) -> int:
    """Nearest E4M3 code, ties to even, saturating at 448."""
    return lib().orc_e4m3_round(v)


def mx_e4m3_quantize(x: np.ndarray):
    """OCP MX quantisation of rows x [rows, n] (n % 32 == 0, any float dtype, taken
    exactly as double) to E4M3 codes [rows, n] and E8M0 scales [rows, n/32]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, n = x.shape
    codes = np.empty((rows, n), np.uint8)
    scales = np.empty((rows, n // 32), np.uint8)
    lib().orc_mx_e4m3_quantize(_p(x), rows, n, _p(codes), _p(scales))
    return codes, scales


def expert_ffn_w4a8(x_rows: np.ndarray, gate, up, down, want_h=False, glu="swiglu"):
    """One expert with MXFP4 weights ((codes, scales) pairs) and MXFP8 activations:
    x_rows bf16 bits [M, D] -> out bf16 bits [M, D] (h [M, I] with want_h)."""
    M, D = x_rows.shape
    (g, gs), (u, us), (d, ds) = gate, up, down
    I = g.shape[0]
    out = np.empty((M, D), np.uint16)
    h = np.empty((M, I), np.uint16) if want_h else None
    lib().orc_expert_ffn_w4a8(_p(np.ascontiguousarray(x_rows, dtype=np.uint16)), M, D, I, _p(g),
                              _p(u), _p(d), _p(gs), _p(us), _p(ds), _p(out), _p(h), GLU[glu])
    return (out, h) if want_h else out


def combine(expert_out, topk_idx, topk_w, pair_row, shared_out, T, k, D):
    y = np.empty((T, D), dtype=expert_out.dtype)
    lib().orc_combine(_p(expert_out), _p(topk_idx), _p(topk_w), _p(pair_row), _p(shared_out),
                      T, k, D, ACT[act_name(expert_out)], _p(y))
    return y


def residual_rmsnorm(x, residual, gamma, eps: float):
    """h = round(x + residual), normed = round(g * h / sqrt(mean(h^2) + eps)) per row.
    Returns (residual_out, normed), both of x's dtype (see orc_residual_rmsnorm)."""
    T, D = x.shape
    assert residual.shape == x.shape and gamma.shape == (D,) and residual.dtype == x.dtype
    res_out = np.empty_like(x)
    normed = np.empty_like(x)
    lib().orc_residual_rmsnorm(_p(x), _p(residual), _p(gamma), eps, T, D, ACT[act_name(x)],
                               _p(res_out), _p(normed))
    return res_out, normed


def combine_rmsnorm(expert_out, topk_idx, topk_w, pair_row, shared_out, residual, gamma, eps,
                    T, k, D):
    """The unfused MoE tail: combine, then the residual add and RMSNorm of its output."""
    y = combine(expert_out, topk_idx, topk_w, pair_row, shared_out, T, k, D)
    return residual_rmsnorm(y, residual, gamma, eps)


def layer_forward(x, token_ids, w_router, bias, experts: dict, shared, T, D, E, k, I,
                  I_shared, mode, wdtype, glu="swiglu"):
    """experts: {e: (gate, up, down)} (entries may be missing for untouched experts;
    mxfp4 entries are (codes, scales) pairs).  shared: (gate, up, down) or None.
    glu: the gated activation of every expert FFN ("swiglu", "clamp", "situ").
    Returns (y, topk_idx, topk_w, macs[3])."""
    arr = ctypes.c_void_p * E
    g, u, d = arr(), arr(), arr()
    gs, us, ds = arr(), arr(), arr()
    keep = []
    for e, (ge, ue, de) in experts.items():
        if wdtype == "mxfp4":
            g[e], gs[e] = _p(ge[0]), _p(ge[1])
            u[e], us[e] = _p(ue[0]), _p(ue[1])
            d[e], ds[e] = _p(de[0]), _p(de[1])
        else:
            g[e], u[e], d[e] = _p(ge), _p(ue), _p(de)
        keep.append((ge, ue, de))
    cast = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
    ex = _Experts(WDT[wdtype], cast(g), cast(u), cast(d),
                  cast(gs) if wdtype == "mxfp4" else None,
                  cast(us) if wdtype == "mxfp4" else None,
                  cast(ds) if wdtype == "mxfp4" else None)
    y = np.empty((T, D), dtype=x.dtype)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    macs = np.zeros(3, dtype=np.uint64)
    sg, su, sd = shared if shared is not None else (None, None, None)
    rc = lib().orc_layer_forward(_p(x), ACT[act_name(x)], _p(token_ids), _p(w_router), _p(bias),
                                 ctypes.byref(ex), _p(sg), _p(su), _p(sd), T, D, E, k, I,
                                 I_shared if shared is not None else 0, ROUTE[mode], _p(y),
                                 _p(idx), _p(w), _p(macs), GLU[glu])
    if rc != 0:
        raise ValueError(f"orc_layer_forward rc={rc}")
    return y, idx, w, macs


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's later calls (the results do not depend on it)."""
    lib().orc_set_num_threads(int(n))
