"""Pins of the oracle's MXFP8 (E4M3 + E8M0 per 32) activation quantisation and
of its FP4 x FP8 expert FFN.

- the E4M3 code table against the OCP FP8 specification's landmark values
  (tests/golden/e4m3_values.txt), and its order;
- rounding: the chosen code is a nearest one, ties go to the even code,
  magnitudes saturate at 448, every finite code rounds to itself;
- block conversion: hand-derived OCP MX cases (tests/golden/mx_e4m3_blocks.txt)
  and the error bound of the format over random blocks;
- the FFN: with activations that MXFP8 holds exactly, the gate/up result is
  the bf16-activation FFN's, bit for bit; the down GEMM sees a quantised h.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


def _f(s):
    return float("nan") if s == "nan" else float.fromhex(s)


def test_e4m3_table_landmarks():
    for ln in read_golden("e4m3_values.txt"):
        code, val = ln.split()
        got, want = oracle.e4m3_value(int(code, 16)), _f(val)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e4m3_table_order_and_symmetry():
    pos = [oracle.e4m3_value(c) for c in range(0x7f)]
    assert all(a < b for a, b in zip(pos, pos[1:]))
    for c in range(0x7f):
        assert oracle.e4m3_value(0x80 | c) == -pos[c]
    # inside each binade the step is 2^(e-10): 8 codes per power of two
    for c in range(8, 0x77):
        assert pos[c + 8] == 2 * pos[c]


def test_e4m3_round_nearest_ties_even_saturate():
    vals = [oracle.e4m3_value(c) for c in range(0x7f)]
    for c, v in enumerate(vals):
        assert oracle.e4m3_round(v) == c
        assert oracle.e4m3_round(-v) == 0x80 | c
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.uniform(0, 448, 2000), np.exp2(rng.uniform(-12, 9, 2000))])
    for x in xs:
        c = oracle.e4m3_round(float(x))
        d = abs(x - vals[c])
        assert all(d <= abs(x - v) for v in vals), x
    # midpoints between neighbours go to the even code
    for c in range(0x7e):
        mid = (vals[c] + vals[c + 1]) / 2
        assert oracle.e4m3_round(mid) == (c if c % 2 == 0 else c + 1)
    assert oracle.e4m3_round(464.0) == 0x7e and oracle.e4m3_round(1e30) == 0x7e
    assert oracle.e4m3_round(-1e30) == 0xfe
    assert oracle.e4m3_round(float("nan")) == 0x7f


def test_mx_block_cases():
    for ln in read_golden("mx_e4m3_blocks.txt"):
        fill, setv, scale, codes = [p.strip() for p in ln.split("|")]
        x = np.full((1, 32), float(fill))
        if setv != "-":
            for item in setv.split():
                i, v = item.split(":")
                x[0, int(i)] = float(v)
        c, s = oracle.mx_e4m3_quantize(x)
        assert int(s[0, 0]) == int(scale), ln
        for item in codes.split():
            i, v = item.split(":")
            assert int(c[0, int(i)]) == int(v, 16), (ln, i)


def test_mx_block_error_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 32)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    c, s = oracle.mx_e4m3_quantize(x)
    for r in range(64):
        X = int(s[r, 0]) - 127
        amax = np.abs(x[r]).max()
        assert 2.0 ** (X + 8) <= amax < 2.0 ** (X + 9)
        for i in range(32):
            deq = oracle.e4m3_value(int(c[r, i])) * 2.0 ** X
            v = x[r, i]
            if abs(v) * 2.0 ** -X > 448:
                assert deq == math.copysign(448 * 2.0 ** X, v)
            else:  # half a step: 2^-4 relative for normals, 2^-10 * 2^X for subnormals
                assert abs(deq - v) <= max(abs(v) * 2.0 ** -4, 2.0 ** (X - 10)) * (1 + 1e-12)


def _mxfp4(rng, rows, cols, lo, hi):
    codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(lo, hi + 1, size=(rows, cols // 32), dtype=np.uint8)
    return packed, scales


def _representable_rows(rng, M, D):
    """bf16 rows that MXFP8 holds exactly: per block an element 256 * 2^X and
    the rest E4M3 codes up to 448, times 2^X."""
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7f)])
    out = np.empty((M, D))
    for r in range(M):
        for b in range(0, D, 32):
            X = int(rng.integers(-12, -4))
            blk = vals[rng.integers(0, 0x7f, 32)] * rng.choice([-1.0, 1.0], 32)
            blk[int(rng.integers(0, 32))] = 256.0
            out[r, b:b + 32] = blk * 2.0 ** X
    return synth.f32_to_bf16(out.astype(np.float32))


def test_w4a8_gate_up_exact_for_representable_activations():
    rng = np.random.default_rng(5)
    M, D, I = 6, 64, 32
    gate, up, down = (_mxfp4(rng, I, D, 118, 124), _mxfp4(rng, I, D, 118, 124),
                      _mxfp4(rng, D, I, 118, 124))
    x = _representable_rows(rng, M, D)
    c, s = oracle.mx_e4m3_quantize((x.astype(np.uint32) << 16).view(np.float32))
    deq = np.array([[oracle.e4m3_value(int(v)) for v in row] for row in c]) * \
        np.exp2(np.repeat(s.astype(np.int64) - 127, 32, axis=1))
    assert np.array_equal(deq, (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    _, h8 = oracle.expert_ffn_w4a8(x, gate, up, down, want_h=True)
    _, h16 = oracle.expert_ffn(x, gate, up, down, "mxfp4", want_h=True)
    assert np.array_equal(h8, h16)


@pytest.mark.parametrize("glu", ["swiglu", "clamp"])
def test_w4a8_ffn_close_to_bf16_activations(glu):
    rng = np.random.default_rng(6)
    M, D, I = 8, 128, 64
    gate, up, down = (_mxfp4(rng, I, D, 120, 124), _mxfp4(rng, I, D, 120, 124),
                      _mxfp4(rng, D, I, 118, 122))
    x = synth.normal_bf16(61, 0, M * D, 1.0).reshape(M, D)
    o8 = oracle.expert_ffn_w4a8(x, gate, up, down, glu=glu)
    o16 = oracle.expert_ffn(x, gate, up, down, "mxfp4", glu=glu)
    f = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rel = np.linalg.norm(f(o8) - f(o16)) / np.linalg.norm(f(o16))
    # E4M3 keeps 4 significant bits (2^-4 relative step): the two quantised GEMMs
    # move the output by a few per cent, and never leave it unchanged
    assert 1e-3 < rel < 0.1, rel


def _bf(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _dequant(codes, scales):
    table = np.array([oracle.e4m3_value(c) for c in range(256)])
    return table[codes] * np.exp2(np.repeat(scales.astype(np.int64) - 127, 32, axis=1))


def _decode_fp4(packed, scales):
    lo, hi = packed & 0xF, packed >> 4
    codes = np.stack([lo, hi], -1).reshape(packed.shape[0], -1)
    table = np.array([[oracle.lib().orc_mxfp4_value(c, s) for s in range(256)] for c in range(16)])
    return table[codes, np.repeat(scales, 32, axis=1)]


def test_w4a8_quantises_both_gemm_inputs():
    rng = np.random.default_rng(7)
    M, D, I = 5, 64, 32
    gate, up, down = (_mxfp4(rng, I, D, 120, 124), _mxfp4(rng, I, D, 120, 124),
                      _mxfp4(rng, D, I, 118, 122))
    x = synth.normal_bf16(62, 0, M * D, 1.0).reshape(M, D)
    o8, h8 = oracle.expert_ffn_w4a8(x, gate, up, down, want_h=True)
    # gate/up: exactly the bf16-activation FFN on the dequantised rows (MXFP8
    # values are bf16 values), and not the FFN on the rows themselves
    xdeq = _dequant(*oracle.mx_e4m3_quantize(_bf(x)))
    _, h_deq = oracle.expert_ffn(synth.f32_to_bf16(xdeq.astype(np.float32)), gate, up, down,
                                 "mxfp4", want_h=True)
    _, h_raw = oracle.expert_ffn(x, gate, up, down, "mxfp4", want_h=True)
    assert np.array_equal(h8, h_deq)
    assert not np.array_equal(h8, h_raw)
    # down: within one rounding of W_down . deq(quant(h)); the unquantised h
    # would land several bf16 steps away
    wd = _decode_fp4(*down)
    hq = _dequant(*oracle.mx_e4m3_quantize(_bf(h8)))
    ref = hq @ wd.T
    got = _bf(o8)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    far = np.abs(_bf(h8) @ wd.T - ref) / np.abs(ref)
    assert far.max() > 2.0 ** -6
