"""Seeded synthetic inputs for the MoE layer (shared by the oracle and the GPU path).

This module produces input tensors only; it contains none of the layer's
arithmetic.  Every tensor is a pure function of (config seed, tensor id,
element index) through the Philox4x32-10 counter-based generator in
``synth.c``, so any slice (one expert's weights, a subset of tokens) can be
generated on its own and is bit-identical to the same slice of the full tensor.

Workload recipes (the five layer shapes this library is measured on):

  1  fp32 tiny:     T=64,   D=256,  E=8,   k=2, I=128,  no shared, softmax routing
                    x, W ~ N(0, 0.02)
  2  bf16 small:    T=512,  D=1024, E=64,  k=6, I=512,  1 shared (I_s=512),
                    sigmoid routing + per-expert bias ~ N(0, 0.01), renormalised
                    x ~ N(0, 1), W ~ N(0, 0.02)
  3  bf16 prefill:  T=4096, D=7168, E=256, k=8, I=2048, 1 shared (I_s=2048),
                    sigmoid routing + Zipf(s=1.1) bias b_e = 0.3 (1+pi(e))^-1.1
                    with pi a seeded permutation; x ~ N(0, 1), W ~ N(0, 0.02)
  4  bf16 decode:   the layer of recipe 3 (same weights), a pool of 64 tokens
                    x ~ N(0, 1) drawn with seed 4; batches T = 1..64
  5  hash + MXFP4:  T=2048, D=7168, E=256, k=8, I=2048, hash routing on token
                    ids uniform in [0, 131072); routed weights N(0, 0.02)
                    quantised to MXFP4 (OCP MX, E2M1 + E8M0 per 32 along K);
                    shared expert (I_s=2048) kept bf16; x ~ N(0, 1) bf16
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

# tensor ids inside one config seed
T_X, T_WR, T_BIAS, T_TOKID, T_PERM = 0, 1, 2, 3, 4
T_SH_GATE, T_SH_UP, T_SH_DOWN = 8, 9, 10


def t_expert(e: int, which: int) -> int:
    """Tensor id of routed expert e's gate (0), up (1) or down (2) matrix."""
    return 16 + 3 * e + which


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        u32, u64, dbl, vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        for name in ("synth_normal_f32", "synth_normal_bf16", "synth_normal_f64"):
            getattr(L, name).argtypes = [u32, u32, u64, u64, dbl, dbl, vp]
            getattr(L, name).restype = None
        L.synth_u32.argtypes = [u32, u32, u64, u64, vp]
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_f32_to_bf16.argtypes = [vp, ctypes.c_int64, vp]
        L.synth_mxfp4_quantize.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def u32(seed, tensor, n, offset=0):
    out = np.empty(n, dtype=np.uint32)
    lib().synth_u32(seed, tensor, offset, n, _ptr(out))
    return out


def normal_f32(seed, tensor, n, std, mean=0.0, offset=0):
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(seed, tensor, offset, n, mean, std, _ptr(out))
    return out


def normal_f64(seed, tensor, n, std, mean=0.0, offset=0):
    out = np.empty(n, dtype=np.float64)
    lib().synth_normal_f64(seed, tensor, offset, n, mean, std, _ptr(out))
    return out


def normal_bf16(seed, tensor, n, std, mean=0.0, offset=0):
    """bf16 bit patterns (uint16) of N(mean, std) rounded fp32 -> bf16 (RNE)."""
    out = np.empty(n, dtype=np.uint16)
    lib().synth_normal_bf16(seed, tensor, offset, n, mean, std, _ptr(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(_ptr(a), a.size, _ptr(out))
    return out


def mxfp4_quantize(w: np.ndarray):
    """OCP MX quantisation of a [rows, cols] fp32 matrix: (codes [rows, cols/2] u8,
    scales [rows, cols/32] u8)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    lib().synth_mxfp4_quantize(_ptr(w), rows, cols, _ptr(codes), _ptr(scales))
    return codes, scales


# ----------------------------------------------------------------------------
# layer recipes

@dataclass(frozen=True)
class LayerConfig:
    cid: int
    name: str
    T: int
    D: int
    E: int
    k: int
    I: int
    I_shared: int  # 0 = no shared expert
    route: str  # "softmax" | "sigmoid" | "hash"
    act: str  # "f32" | "bf16"
    wdtype: str  # "f32" | "bf16" | "mxfp4" (routed experts)
    x_std: float
    w_std: float
    bias: str  # "none" | "normal" | "zipf"
    bias_std: float = 0.0
    seed: int = 0
    weight_seed: int = 0  # seed of the weights (recipe 4 shares recipe 3's layer)

    def with_T(self, T: int) -> "LayerConfig":
        d = dict(self.__dict__)
        d["T"] = T
        return LayerConfig(**d)


CONFIGS = {
    1: LayerConfig(1, "tiny-fp32", 64, 256, 8, 2, 128, 0, "softmax", "f32", "f32",
                   0.02, 0.02, "none", seed=1, weight_seed=1),
    2: LayerConfig(2, "small-bf16", 512, 1024, 64, 6, 512, 512, "sigmoid", "bf16", "bf16",
                   1.0, 0.02, "normal", 0.01, seed=2, weight_seed=2),
    3: LayerConfig(3, "dsv3-prefill-bf16", 4096, 7168, 256, 8, 2048, 2048, "sigmoid", "bf16",
                   "bf16", 1.0, 0.02, "zipf", seed=3, weight_seed=3),
    4: LayerConfig(4, "dsv3-decode-bf16", 64, 7168, 256, 8, 2048, 2048, "sigmoid", "bf16",
                   "bf16", 1.0, 0.02, "zipf", seed=4, weight_seed=3),
    5: LayerConfig(5, "hash-mxfp4", 2048, 7168, 256, 8, 2048, 2048, "hash", "bf16", "mxfp4",
                   1.0, 0.02, "none", seed=5, weight_seed=5),
}

TOKEN_ID_RANGE = 131072


def x_tokens(cfg: LayerConfig, T: int | None = None, offset_tokens: int = 0):
    """Activations [T, D]: float32 array for f32 recipes, uint16 bf16 bits otherwise."""
    T = cfg.T if T is None else T
    n = T * cfg.D
    off = offset_tokens * cfg.D
    if cfg.act == "f32":
        return normal_f32(cfg.seed, T_X, n, cfg.x_std, offset=off).reshape(T, cfg.D)
    return normal_bf16(cfg.seed, T_X, n, cfg.x_std, offset=off).reshape(T, cfg.D)


def token_ids(cfg: LayerConfig, T: int | None = None, offset_tokens: int = 0):
    T = cfg.T if T is None else T
    r = u32(cfg.seed, T_TOKID, T, offset=offset_tokens)
    return (r >> np.uint32(15)).astype(np.int32)  # uniform in [0, 131072)


def router_weight(cfg: LayerConfig):
    n = cfg.E * cfg.D
    s = cfg.weight_seed
    if cfg.act == "f32":
        return normal_f32(s, T_WR, n, cfg.w_std).reshape(cfg.E, cfg.D)
    return normal_bf16(s, T_WR, n, cfg.w_std).reshape(cfg.E, cfg.D)


def seeded_permutation(seed: int, tensor: int, n: int) -> np.ndarray:
    """Fisher–Yates shuffle of 0..n-1 driven by Philox draws (modulo bias is
    irrelevant for input generation)."""
    r = u32(seed, tensor, n)
    p = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = int(r[i]) % (i + 1)
        p[i], p[j] = p[j], p[i]
    return p


def router_bias(cfg: LayerConfig):
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal":
        return normal_f32(cfg.weight_seed, T_BIAS, cfg.E, cfg.bias_std)
    if cfg.bias == "zipf":
        pi = seeded_permutation(cfg.weight_seed, T_PERM, cfg.E)
        return (0.3 * (1.0 + pi.astype(np.float64)) ** -1.1).astype(np.float32)
    raise ValueError(cfg.bias)


def _matrix(cfg: LayerConfig, tensor: int, rows: int, cols: int, kind: str):
    n = rows * cols
    s = cfg.weight_seed
    if kind == "f32":
        return normal_f32(s, tensor, n, cfg.w_std).reshape(rows, cols)
    if kind == "bf16":
        return normal_bf16(s, tensor, n, cfg.w_std).reshape(rows, cols)
    if kind == "mxfp4":
        return mxfp4_quantize(normal_f32(s, tensor, n, cfg.w_std).reshape(rows, cols))
    raise ValueError(kind)


def expert_matrices(cfg: LayerConfig, e: int):
    """(gate [I,D], up [I,D], down [D,I]) of routed expert e in cfg.wdtype.
    For mxfp4 each entry is a (codes, scales) pair."""
    I, D = cfg.I, cfg.D
    return (_matrix(cfg, t_expert(e, 0), I, D, cfg.wdtype),
            _matrix(cfg, t_expert(e, 1), I, D, cfg.wdtype),
            _matrix(cfg, t_expert(e, 2), D, I, cfg.wdtype))


def shared_matrices(cfg: LayerConfig):
    """(gate [I_s,D], up [I_s,D], down [D,I_s]); bf16 even when routed experts are
    MXFP4 (the shared expert is kept at the higher precision)."""
    if cfg.I_shared == 0:
        return None
    kind = "f32" if cfg.act == "f32" else "bf16"
    Is, D = cfg.I_shared, cfg.D
    return (_matrix(cfg, T_SH_GATE, Is, D, kind),
            _matrix(cfg, T_SH_UP, Is, D, kind),
            _matrix(cfg, T_SH_DOWN, D, Is, kind))
