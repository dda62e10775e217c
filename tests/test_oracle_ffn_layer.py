"""Pins of the oracle's expert FFN, combine and whole layer.

- SwiGLU: the worked example of the forum article (section "SiTU-GLU":
  Swish(20) * 30 is about 600) and silu(0) = 0;
- dense special case (E=1, k=1): the layer reduces to one SwiGLU FFN, checked
  against an independent numpy float64 matmul implementation (the rounding
  points differ, so within a derived tolerance);
- FLOPs scale with k, not E (forum article, section on MoE FLOPs): the oracle's
  executed multiply-add counters;
- k = E with identical experts: y equals the single FFN;
- combine order: hand-derived golden cases;
- MXFP4 expert equals the bf16 expert on the dequantized weights, bitwise;
- batch invariance: a token's output is the same alone or in any batch.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


def bf16_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16(a):
    return synth.f32_to_bf16(np.asarray(a, dtype=np.float32))


def test_swiglu_worked_example():
    (g, u, approx, tol), = [list(map(float, ln.split())) for ln in read_golden("swiglu_worked_example.txt")]
    D, I = 32, 1
    for act in ("f32", "bf16"):
        x = np.zeros((1, D), dtype=np.float32)
        x[0, 0] = 1.0
        wg = np.zeros((I, D), np.float32)
        wu = np.zeros((I, D), np.float32)
        wd = np.zeros((D, I), np.float32)
        wg[0, 0], wu[0, 0], wd[0, 0] = g, u, 1.0
        if act == "bf16":
            x, wg, wu, wd = map(to_bf16, (x, wg, wu, wd))
        out, h = oracle.expert_ffn(x, wg, wu, wd, act, want_h=True)
        hv = float(h[0, 0]) if act == "f32" else float(bf16_to_f64(h[0, 0]))
        assert abs(hv - approx) <= tol
        assert hv == pytest.approx(g * u / (1 + math.exp(-g)), rel=1e-6 if act == "f32" else 4e-3)
        ov = float(out[0, 0]) if act == "f32" else float(bf16_to_f64(out[0, 0]))
        assert ov == hv
        # silu(0) = 0 whatever the up branch
        wg[...] = 0
        out0 = oracle.expert_ffn(x, wg, wu, wd, act)
        assert np.all((out0 if act == "f32" else bf16_to_f64(out0)) == 0)


def _numpy_ffn(x, wg, wu, wd):
    g = x @ wg.T
    u = x @ wu.T
    return (g / (1 + np.exp(-g)) * u) @ wd.T


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_dense_special_case_matches_numpy(act):
    rng = np.random.default_rng(5)
    T, D, I = 24, 96, 64  # I != D so a transposed operand cannot pass
    x = rng.standard_normal((T, D)).astype(np.float32)
    wg, wu = (0.1 * rng.standard_normal((2, I, D))).astype(np.float32)
    wd = (0.1 * rng.standard_normal((D, I))).astype(np.float32)
    wr = (0.02 * rng.standard_normal((1, D))).astype(np.float32)
    if act == "bf16":
        xs, wgs, wus, wds, wrs = map(to_bf16, (x, wg, wu, wd, wr))
        xf, wgf, wuf, wdf = map(bf16_to_f64, (xs, wgs, wus, wds))
    else:
        xs, wgs, wus, wds, wrs = x, wg, wu, wd, wr
        xf, wgf, wuf, wdf = (a.astype(np.float64) for a in (x, wg, wu, wd))
    y, idx, w, macs = oracle.layer_forward(xs, None, wrs, None, {0: (wgs, wus, wds)}, None,
                                           T, D, 1, 1, I, 0, "softmax", act)
    assert np.all(idx == 0) and np.all(w == 1.0)
    ref = _numpy_ffn(xf, wgf, wuf, wdf)
    got = y.astype(np.float64) if act == "f32" else bf16_to_f64(y)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    # fp32: two fp32 roundings (h, y); bf16: roundings of h and y at 2^-9 each
    assert rel <= (1e-6 if act == "f32" else 4e-3), rel
    assert rel > 0 or act == "f32"


def test_macs_scale_with_k_not_E():
    rng = np.random.default_rng(6)
    T, D, I, k = 16, 64, 32, 2
    x = to_bf16(rng.standard_normal((T, D)))
    got = {}
    for E in (4, 8, 16):
        wr = to_bf16(0.02 * rng.standard_normal((E, D)))
        ex = {e: tuple(to_bf16(0.02 * rng.standard_normal(s)) for s in ((I, D), (I, D), (D, I)))
              for e in range(E)}
        _, _, _, macs = oracle.layer_forward(x, None, wr, None, ex, None, T, D, E, k, I, 0,
                                             "sigmoid", "bf16")
        assert int(macs[1]) == T * k * 3 * D * I  # routed expert work: k, not E
        assert int(macs[0]) == T * E * D           # router: grows with E
        got[E] = int(macs[1])
    assert len(set(got.values())) == 1


def test_k_equals_E_identical_experts():
    rng = np.random.default_rng(7)
    T, D, I, E = 8, 64, 32, 4
    x = rng.standard_normal((T, D)).astype(np.float32)
    wr = (0.5 * rng.standard_normal((E, D))).astype(np.float32)
    m = tuple((0.1 * rng.standard_normal(s)).astype(np.float32) for s in ((I, D), (I, D), (D, I)))
    y, _, w, _ = oracle.layer_forward(x, None, wr, None, {e: m for e in range(E)}, None,
                                      T, D, E, E, I, 0, "softmax", "f32")
    single = oracle.expert_ffn(x, *m, "f32")
    # sum_e w_e * o = o * sum_e w_e, with sum w = 1 up to fp32 rounding
    assert np.allclose(y, single, rtol=4e-6, atol=1e-9)


def test_combine_order_golden():
    for ln in read_golden("combine_order.txt"):
        lhs, rhs = ln.split("=")
        parts = [p.split() for p in lhs.split("|")]
        k = int(parts[0][0])
        ids = np.array([int(v) for v in parts[0][1:]], dtype=np.int32).reshape(1, k)
        fv = lambda s: float.fromhex(s) if "0x" in s else float(s)
        w = np.array([fv(v) for v in parts[1]], dtype=np.float32).reshape(1, k)
        o = np.array([fv(v) for v in parts[2]], dtype=np.float32).reshape(k, 1)
        s = None if parts[3][0] == "-" else np.array([[fv(parts[3][0])]], dtype=np.float32)
        pair_row = np.arange(k, dtype=np.int32)
        y = oracle.combine(o, ids, w, pair_row, s, 1, k, 1)
        assert y[0, 0] == np.float32(float.fromhex(rhs.strip())), ln


def test_mxfp4_equals_bf16_on_dequantized():
    rng = np.random.default_rng(8)
    M, D, I = 5, 64, 32
    x = to_bf16(rng.standard_normal((M, D)))
    q = [synth.mxfp4_quantize((0.02 * rng.standard_normal(s)).astype(np.float32))
         for s in ((I, D), (I, D), (D, I))]
    deq = []
    for codes, scales in q:
        rows, half = codes.shape
        vals = np.empty((rows, half * 2))
        for r in range(rows):
            for c in range(half * 2):
                b = codes[r, c // 2]
                code = (b >> 4) if c & 1 else (b & 0xF)
                vals[r, c] = oracle.lib().orc_mxfp4_value(int(code), int(scales[r, c // 32]))
        deq.append(to_bf16(vals))
        assert np.array_equal(bf16_to_f64(deq[-1]), vals)  # exact in bf16
    a = oracle.expert_ffn(x, *q, "mxfp4")
    b = oracle.expert_ffn(x, *deq, "bf16")
    assert np.array_equal(a, b)


def test_oracle_batch_invariance():
    cfg = synth.CONFIGS[2].with_T(40)
    x = synth.x_tokens(cfg)
    ex = {e: synth.expert_matrices(cfg, e) for e in range(cfg.E)}
    args = (synth.router_weight(cfg), synth.router_bias(cfg), ex, synth.shared_matrices(cfg))
    y_all, idx_all, w_all, _ = oracle.layer_forward(
        x, None, args[0], args[1], args[2], args[3], cfg.T, cfg.D, cfg.E, cfg.k, cfg.I,
        cfg.I_shared, cfg.route, cfg.wdtype)
    perm = np.random.default_rng(9).permutation(cfg.T)[:7]
    y_sub, idx_sub, _, _ = oracle.layer_forward(
        np.ascontiguousarray(x[perm]), None, args[0], args[1], args[2], args[3], len(perm),
        cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.route, cfg.wdtype)
    assert np.array_equal(y_sub, y_all[perm])
    assert np.array_equal(idx_sub, idx_all[perm])


def test_oracle_vs_independent_fp32_error_scale():
    """An fp32 implementation that keeps no bf16 intermediates differs from the
    oracle by about the bf16 rounding of h, o and y: rel-L2 around 1e-3."""
    cfg = synth.CONFIGS[2].with_T(32)
    x = synth.x_tokens(cfg)
    wr, bias = synth.router_weight(cfg), synth.router_bias(cfg)
    ex = {e: synth.expert_matrices(cfg, e) for e in range(cfg.E)}
    sh = synth.shared_matrices(cfg)
    y, idx, w, _ = oracle.layer_forward(x, None, wr, bias, ex, sh, cfg.T, cfg.D, cfg.E, cfg.k,
                                        cfg.I, cfg.I_shared, cfg.route, cfg.wdtype)
    xf = bf16_to_f64(x).astype(np.float32)
    ref = np.zeros((cfg.T, cfg.D), np.float32)
    for t in range(cfg.T):
        for j in range(cfg.k):
            m = [bf16_to_f64(a).astype(np.float32) for a in ex[int(idx[t, j])]]
            ref[t] += w[t, j] * _numpy_ffn(xf[t:t + 1], *m)[0].astype(np.float32)
    ref += _numpy_ffn(xf, *[bf16_to_f64(a).astype(np.float32) for a in sh]).astype(np.float32)
    rel = np.linalg.norm(bf16_to_f64(y) - ref) / np.linalg.norm(ref)
    assert 1e-4 < rel < 4e-3, rel
