"""FP4 x FP8 (W4A8) expert compute on the GPU (through the C-ABI): MXFP8
activation quantisation and the grouped FFN on gfx950's scaled MFMA.

- quantisation: codes and scales bit-exact against the oracle over all 65536
  bf16 bit patterns (in sorted and shuffled blocks), zero / tiny / huge /
  non-finite blocks, and through a row index;
- the grouped FFN against the oracle's FP4 x FP8 FFN expert by expert (an
  empty expert, ragged row tiles), with each gated activation;
- a row's output is the same bits in any batch.
"""
import numpy as np
import pytest
import torch

import invariant_moe_amd as moe
import oracle
import synth
from gpu_util import banner, dev, rel_l2, requires_gpu, to_np

pytestmark = [pytest.mark.gpu, requires_gpu]


def _f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _check_quant(x_bits, row_index=None):
    xg = x_bits if row_index is None else x_bits[row_index]
    c_ref, s_ref = oracle.mx_e4m3_quantize(_f64(xg))
    c, s = moe.mx_e4m3_quantize(dev(x_bits), dev(row_index) if row_index is not None else None)
    c, s = to_np(c), to_np(s)
    bad = np.nonzero(c != c_ref)
    assert np.array_equal(s, s_ref), np.nonzero(s != s_ref)[0][:5]
    assert bad[0].size == 0, [(int(r), int(k), hex(xg[r, k]), int(c[r, k]), int(c_ref[r, k]))
                              for r, k in zip(*[a[:5] for a in bad])]


def test_quantize_every_bf16_pattern():
    banner("mx e4m3 quantize: all bf16 patterns")
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    # sorted by magnitude (blocks of neighbouring values: every exponent, ties,
    # subnormal edges), then shuffled (wide blocks: saturation, underflow)
    order = np.argsort(np.abs(_f64(allv)), kind="stable")
    _check_quant(np.ascontiguousarray(allv[order].reshape(-1, 256)))
    rng = np.random.default_rng(90)
    _check_quant(np.ascontiguousarray(rng.permutation(allv).reshape(-1, 1024)))


def test_quantize_special_blocks_and_row_index():
    banner("mx e4m3 quantize: special blocks")
    rng = np.random.default_rng(91)
    rows = []
    for sc in (2.0 ** -140, 2.0 ** -125, 2.0 ** -20, 1.0, 2.0 ** 20, 2.0 ** 120):
        rows.append(rng.standard_normal(128) * sc)
    rows.append(np.zeros(128))
    r = rng.standard_normal(128)
    r[3], r[40], r[77] = np.inf, -np.inf, np.nan  # non-finite values in three blocks
    rows.append(r)
    x = synth.f32_to_bf16(np.array(rows, np.float32))
    _check_quant(x)
    _check_quant(x, np.array([7, 0, 3, 3, 5, 1], np.int32))


def _mxfp4(rng, shape, lo, hi):
    codes = rng.integers(0, 16, size=shape, dtype=np.uint8)
    scales = rng.integers(lo, hi + 1, size=shape[:-1] + (shape[-1] // 32,), dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8), scales


def _experts(seed, E, D, I):
    rng = np.random.default_rng(seed)
    return [_mxfp4(rng, (E, I, D), 120, 124), _mxfp4(rng, (E, I, D), 120, 124),
            _mxfp4(rng, (E, D, I), 118, 122)]


@pytest.mark.parametrize("glu", ["swiglu", "clamp", "situ"])
def test_grouped_ffn_w4a8_vs_oracle(glu):
    banner(f"w4a8 grouped FFN glu={glu}")
    E, D, I = 6, 384, 256
    counts = np.array([70, 0, 1, 64, 129, 17], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    m = _experts(92, E, D, I)
    x = synth.normal_bf16(93, 0, 300 * D, 1.0).reshape(300, D)
    row_index = np.random.default_rng(94).integers(0, 300, R).astype(np.int32)
    w = moe.ExpertWeights(*(dev(a[0]) for a in m), *(dev(a[1]) for a in m))
    out = to_np(moe.grouped_swiglu_w4a8(dev(x), dev(row_index), dev(offsets), R, E, w, glu=glu))
    ref = np.empty_like(out)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            ref[a:b] = oracle.expert_ffn_w4a8(np.ascontiguousarray(x[row_index[a:b]]),
                                              *[(a_[0][e], a_[1][e]) for a_ in m], glu=glu)
    r = rel_l2(out, ref)
    banner(f"w4a8 {glu} rel_l2={r:.3e}, equal {np.mean(out == ref):.4f}")
    assert r <= 2e-3, r
    assert ((out & 0x7F80) != 0x7F80).all()


def test_grouped_ffn_w4a8_rows_equal_in_any_batch():
    """100 rows per expert take 128 x 128 tiles, 20 rows 64 x 128, 0 rows 64 x 64:
    the same bits in each."""
    banner("w4a8 batch invariance")
    E, D, I = 4, 256, 128
    m = _experts(95, E, D, I)
    w = moe.ExpertWeights(*(dev(a[0]) for a in m), *(dev(a[1]) for a in m))
    x = synth.normal_bf16(96, 0, 400 * D, 1.0).reshape(400, D)
    full_counts = np.array([150, 3, 200, 47], np.int32)
    off = np.concatenate([[0], np.cumsum(full_counts)]).astype(np.int32)
    full = to_np(moe.grouped_swiglu_w4a8(dev(x), None, dev(off), 400, E, w))
    for keep in (np.array([150, 3, 200, 47]), np.array([1, 0, 65, 16]), np.array([0, 0, 1, 0])):
        sub_rows = np.concatenate([np.arange(off[e], off[e] + keep[e]) for e in range(E)])
        sub_off = np.concatenate([[0], np.cumsum(keep)]).astype(np.int32)
        got = to_np(moe.grouped_swiglu_w4a8(dev(x), dev(sub_rows.astype(np.int32)), dev(sub_off),
                                            len(sub_rows), E, w))
        assert np.array_equal(got, full[sub_rows]), keep


def test_layer_w4a8_vs_composed_oracle_and_invariance():
    """moe_layer_forward with MOE_FLAG_W4A8: routing, the FP4 x FP8 routed
    experts, the bf16 shared expert and the combine, against the oracle's
    stages composed; a token's row is the same bits at every T, across the
    three FP4 x FP8 tile shapes and the shared expert's 128- and 64-row
    bf16 tiles."""
    banner("w4a8 layer")
    E, k, D, I, Is, T = 8, 2, 256, 128, 128, 400  # 100 rows per expert: 128-row tiles
    m = _experts(97, E, D, I)
    sh = [synth.normal_bf16(98, t, n, 0.05).reshape(shape)
          for t, (n, shape) in enumerate(((Is * D, (Is, D)), (Is * D, (Is, D)), (D * Is, (D, Is))))]
    wr = synth.normal_bf16(99, 0, E * D, 0.05).reshape(E, D)
    x = synth.normal_bf16(100, 0, T * D, 1.0).reshape(T, D)
    routed = moe.ExpertWeights(*(dev(a[0]) for a in m), *(dev(a[1]) for a in m))
    shared = moe.ExpertWeights(*(dev(a[None]) for a in sh))
    layer = moe.MoELayer(dev(wr), None, routed, shared, E, k, "softmax", w4a8=True)
    y = to_np(layer.forward(dev(x)))
    idx, w = oracle.route(oracle.router_logits(x, wr), None, None, T, E, k, "softmax")
    _, offsets, row_token, pair_row = oracle.permute(idx, E)
    o_ref = np.empty((T * k, D), np.uint16)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            o_ref[a:b] = oracle.expert_ffn_w4a8(np.ascontiguousarray(x[row_token[a:b]]),
                                                *[(a_[0][e], a_[1][e]) for a_ in m])
    s_ref = oracle.expert_ffn(x, *sh, "bf16")
    y_ref = oracle.combine(o_ref, idx, w, pair_row, s_ref, T, k, D)
    r = rel_l2(y, y_ref)
    banner(f"w4a8 layer rel_l2={r:.3e}")
    assert r <= 2e-3, r
    # not the W4A16 layer: the activations were quantised
    plain = to_np(moe.MoELayer(dev(wr), None, routed, shared, E, k, "softmax").forward(dev(x)))
    assert not np.array_equal(plain, y)
    for t in (150, 37, 5, 1):  # 64-row tiles
        assert np.array_equal(to_np(layer.forward(dev(np.ascontiguousarray(x[:t])))), y[:t]), t
