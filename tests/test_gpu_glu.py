"""Gated-activation variants of the expert FFN on the GPU (through the C-ABI):
the clamped SwiGLU (MOE_FLAG_GLU_CLAMP) and SiTU-GLU (MOE_FLAG_GLU_SITU).

- the whole layer, routed and shared experts, against the oracle for bf16,
  MXFP4 and fp32 weights, with branch values large enough that the caps act;
- the grouped expert FFN entry point against the oracle's expert FFN, with an
  empty expert and a ragged tail;
- every row-tile bracket gives the same bits for a token at every T, and MXFP4
  weights the bits of bf16 weights decoded from them.
"""
import numpy as np
import pytest

import invariant_moe_amd as moe
import oracle
import synth
from gpu_util import (banner, dev, mxfp4_decode_bf16, mxfp4_pack, rel_l2, requires_gpu, to_np,
                      tol_for)

pytestmark = [pytest.mark.gpu, requires_gpu]

E, K, D, I, IS = 8, 2, 288, 96, 64  # K % 64 == 32 in both GEMMs (trailing half step)
GU_STD = 0.7                          # gate/up branch values ~ N(0, 12^2): past both caps
DN_STD = 0.05


def _normal(act, seed, tensor, shape, std):
    n = int(np.prod(shape))
    if act == "f32":
        return synth.normal_f32(seed, tensor, n, std).reshape(shape)
    return synth.normal_bf16(seed, tensor, n, std).reshape(shape)


def _dense(act, seed, G, i_dim):
    return (_normal(act, seed, 0, (G, i_dim, D), GU_STD),
            _normal(act, seed, 1, (G, i_dim, D), GU_STD),
            _normal(act, seed, 2, (G, D, i_dim), DN_STD))


def _mxfp4(rng, shape, lo, hi):
    codes = rng.integers(0, 16, size=shape, dtype=np.uint8)
    scales = rng.integers(lo, hi + 1, size=(shape[0], shape[1], shape[2] // 32), dtype=np.uint8)
    packed = mxfp4_pack(codes)
    return packed, scales


def _mxfp4_routed(seed):
    # E2M1 codes have RMS ~2.9: scales 2^-3..2^-1 give gate/up branches of
    # order 10 at D = 288; down scales 2^-9..2^-6.
    rng = np.random.default_rng(seed)
    return [_mxfp4(rng, (E, I, D), 124, 126), _mxfp4(rng, (E, I, D), 124, 126),
            _mxfp4(rng, (E, D, I), 118, 121)]


def _weights_dev(m, fp4):
    if fp4:
        return moe.ExpertWeights(*(dev(a[0]) for a in m), *(dev(a[1]) for a in m))
    return moe.ExpertWeights(*(dev(a) for a in m))


def _oracle_experts(m, fp4):
    if fp4:
        return {e: tuple((np.ascontiguousarray(a[0][e]), np.ascontiguousarray(a[1][e]))
                         for a in m) for e in range(E)}
    return {e: tuple(np.ascontiguousarray(a[e]) for a in m) for e in range(E)}


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "f32"])
@pytest.mark.parametrize("glu", ["clamp", "situ", "swiglu"])
def test_layer_variant_vs_oracle(glu, fmt):
    act = "f32" if fmt == "f32" else "bf16"
    T = 150
    banner(f"layer glu={glu} weights={fmt} T={T}")
    fp4 = fmt == "mxfp4"
    routed = _mxfp4_routed(41) if fp4 else _dense(act, 41, E, I)
    shared = _dense(act, 42, 1, IS)
    w_router = _normal(act, 43, 0, (E, D), 0.05)
    x = _normal(act, 44, 0, (T, D), 1.0)
    layer = moe.MoELayer(dev(w_router), None, _weights_dev(routed, fp4), _weights_dev(shared, False),
                         E, K, "softmax", glu=glu)
    y = to_np(layer.forward(dev(x)))
    sh = tuple(np.ascontiguousarray(a[0]) for a in shared)
    y_ref, _, _, _ = oracle.layer_forward(x, None, w_router, None, _oracle_experts(routed, fp4), sh,
                                          T, D, E, K, I, IS, "softmax", fmt, glu=glu)
    r = rel_l2(y, y_ref)
    banner(f"glu={glu} {fmt} rel_l2={r:.3e}")
    assert r <= tol_for(act), r
    if glu != "swiglu":  # the caps changed the layer output
        y_plain, _, _, _ = oracle.layer_forward(x, None, w_router, None,
                                                _oracle_experts(routed, fp4), sh, T, D, E, K, I,
                                                IS, "softmax", fmt)
        assert rel_l2(y_plain, y_ref) > 0.05


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("glu", ["clamp", "situ"])
def test_grouped_ffn_variant_vs_oracle(glu, act):
    banner(f"grouped FFN glu={glu} act={act}")
    counts = np.array([37, 0, 5, 64, 1, 90, 16, 3], np.int32)  # an empty expert, ragged tiles
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    m = _dense(act, 51, E, I)
    x = _normal(act, 52, 0, (R, D), 1.0)
    out = to_np(moe.grouped_swiglu(dev(x), None, dev(offsets), R, E, _weights_dev(m, False),
                                   glu=glu))
    ref = np.empty_like(out)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            ref[a:b] = oracle.expert_ffn(np.ascontiguousarray(x[a:b]), m[0][e], m[1][e], m[2][e],
                                         act, glu=glu)
    r = rel_l2(out, ref)
    banner(f"grouped glu={glu} {act} rel_l2={r:.3e}")
    assert r <= tol_for(act), r


@pytest.mark.parametrize("glu", ["clamp", "situ"])
def test_variant_bitwise_across_tiles_and_formats(glu):
    """Rows per expert T*k/E = 150, 37.5, 5, 0.75, 0.25 cover every row-tile
    bracket; MXFP4 routed experts give the bits of their decoded bf16 weights."""
    banner(f"glu={glu} tile brackets x formats")
    routed = _mxfp4_routed(61)
    dec = [mxfp4_decode_bf16(p, s) for p, s in routed]
    shared = _dense("bf16", 62, 1, IS)
    w_router = dev(_normal("bf16", 63, 0, (E, D), 0.05))
    sh = _weights_dev(shared, False)
    l4 = moe.MoELayer(w_router, None, _weights_dev(routed, True), sh, E, K, "softmax", glu=glu)
    l16 = moe.MoELayer(w_router, None, _weights_dev(dec, False), sh, E, K, "softmax", glu=glu)
    lplain = moe.MoELayer(w_router, None, _weights_dev(dec, False), sh, E, K, "softmax")
    xs = _normal("bf16", 64, 0, (600, D), 1.0)
    y_all = None
    for T in (600, 150, 20, 3, 1):
        x = dev(np.ascontiguousarray(xs[:T]))
        y4, y16 = to_np(l4.forward(x)), to_np(l16.forward(x))
        assert np.array_equal(y4, y16), T
        if y_all is None:
            y_all = y16
            assert ((y_all & 0x7F80) != 0x7F80).all()  # finite bf16
            assert not np.array_equal(y_all, to_np(lplain.forward(x)))
        else:
            assert np.array_equal(y16, y_all[:T]), T
