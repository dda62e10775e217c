"""Pins of the oracle's scalar numerics against mathematics and libraries.

exp / sigmoid: the routing exp is this library's own definition (Cody–Waite +
Taylor in fp32); it is pinned to the true exponential (numpy float64) within
2 ulp, and the sigmoid within 4 ulp.
bf16 rounding: pinned to hand-derived ties and to torch's fp32->bf16 RNE.
MXFP4: pinned exhaustively to the OCP MX E2M1 value table, and to the
DeepSeek-V4 infra walkthrough's claim (section 6.2) that E2M1 values times the
block scale are exact in FP8 — within the scale windows where that holds.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def _ulp32(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(np.maximum(e, -126.0) - 23.0)


def _f32_range(lo: float, hi: float, stride: int) -> np.ndarray:
    """Every `stride`-th fp32 value in [lo, hi] (by bit pattern)."""
    def key(v):  # monotone int key of a float32
        b = np.array([v], dtype=np.float32).view(np.int32)[0]
        return int(b) if b >= 0 else -(int(b) & 0x7FFFFFFF)
    ks = np.arange(key(lo), key(hi) + 1, stride, dtype=np.int64)
    bits = np.where(ks >= 0, ks, (-ks) | 0x80000000).astype(np.uint32)
    return bits.view(np.float32)


def test_exp_special_values():
    assert oracle.exp(0.0) == 1.0
    assert oracle.exp(-0.0) == 1.0
    assert math.isinf(oracle.exp(89.5)) and math.isinf(oracle.exp(1e30))
    assert oracle.exp(-104.5) == 0.0 and oracle.exp(-1e30) == 0.0
    assert math.isnan(oracle.exp(float("nan")))
    assert math.isinf(oracle.exp(88.72284))  # above ln(FLT_MAX) = 88.7228391...
    assert oracle.exp(88.7228) < 3.4028235e38


@pytest.mark.parametrize("lo,hi,stride", [(-103.0, 88.72, 997), (-1.0, 1.0, 61),
                                          (-0.01, 0.01, 7)])
def test_exp_within_2ulp(lo, hi, stride):
    x = _f32_range(lo, hi, stride)
    got = oracle.exp_array(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    err = np.abs(got - ref) / _ulp32(ref)
    assert err.max() <= 2.0, (x[err.argmax()], err.max())


def test_exp_subnormal_results():
    x = _f32_range(-103.97, -87.4, 13)
    got = oracle.exp_array(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    err = np.abs(got - ref) / _ulp32(ref)  # ulp is 2^-149 below 2^-126
    assert err.max() <= 2.0


def test_exp_monotone():
    x = _f32_range(-20.0, 20.0, 1013)
    y = oracle.exp_array(x)
    assert np.all(np.diff(y.astype(np.float64)) >= 0)


def test_sigmoid_values():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(200.0) == 1.0
    assert oracle.sigmoid(-200.0) == 0.0
    x = _f32_range(-80.0, 80.0, 509)
    got = oracle.sigmoid_array(x).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    nz = ref > 1e-37
    err = np.abs(got - ref)[nz] / _ulp32(ref[nz])
    assert err.max() <= 4.0
    assert np.all(np.diff(got) >= 0)


def test_bf16_rounding_hand_cases():
    c = oracle.lib().orc_bf16_from_f64
    assert c(1.0) == 0x3F80
    assert c(1.0 + 2**-8) == 0x3F80           # tie -> even (down)
    assert c(1.0 + 3 * 2**-8) == 0x3F82       # tie -> even (up)
    assert c(1.0 + 2**-8 + 2**-40) == 0x3F81  # just above the tie: one rounding, up
    # the same value through fp32 first would be a tie and go down: double rounding
    assert oracle.lib().orc_bf16_from_f32(float(np.float32(1.0 + 2**-8 + 2**-40))) == 0x3F80
    assert c(-2.0) == 0xC000
    assert c(0.0) == 0x0000 and c(-0.0) == 0x8000
    assert c(3.5e38) == 0x7F80                # above bf16 max + half ulp -> inf
    assert c(2.0**-133) == 0x0001             # smallest bf16 subnormal
    assert c(2.0**-134) == 0x0000             # tie with 0 -> even
    assert c(3 * 2.0**-134) == 0x0002         # tie between 1 and 2 quanta -> even
    assert c(600.0) == 0x4416
    n = c(float("nan"))
    assert n & 0x7F80 == 0x7F80 and n & 0x007F != 0  # a NaN stays a NaN


def test_bf16_rounding_matches_torch_on_fp32():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    got = oracle.bf16_from_f64_array(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# OCP MX v1.0 E2M1 element values (codes 0..7; codes 8..15 are their negatives)
OCP_E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
            Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def test_mxfp4_decode_exhaustive():
    for s in range(255):
        for code in range(16):
            ref = OCP_E2M1[code & 7] * (Fraction(2) ** (s - 127))
            if code & 8:
                ref = -ref
            got = oracle.lib().orc_mxfp4_value(code, s)
            assert Fraction(got) == ref, (code, s)
    assert math.isnan(oracle.lib().orc_mxfp4_value(1, 255))


def _representable(v: Fraction, mant_bits: int, emin: int, emax_value: Fraction) -> bool:
    """Exact in a binary float format with `mant_bits` stored mantissa bits,
    normal exponent >= emin (subnormals below), largest finite value emax_value."""
    if v == 0:
        return True
    a = abs(v)
    if a > emax_value:
        return False
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, emin) - mant_bits)
    return (a / q).denominator == 1


E4M3_MAX = Fraction(448)
E5M2_MAX = Fraction(57344)
BF16_MAX = Fraction(2) ** 127 * (2 - Fraction(1, 2**7))


def test_fp4_times_scale_exact_windows():
    """FP4 (E2M1) x block scale is exact in FP8 (DeepSeek-V4 infra, 6.2) — true
    for E4M3 iff the scale exponent is in [-8, 6], for E5M2 iff in [-15, 13],
    and in bf16 iff it is <= 125."""
    for s in range(-127, 128):
        vals = [OCP_E2M1[c] * Fraction(2) ** s for c in range(8)]
        e4 = all(_representable(v, 3, -6, E4M3_MAX) for v in vals)
        e5 = all(_representable(v, 2, -14, E5M2_MAX) for v in vals)
        bf = all(_representable(v, 7, -126, BF16_MAX) for v in vals)
        assert e4 == (-8 <= s <= 6), s
        assert e5 == (-15 <= s <= 13), s
        assert bf == (s <= 125), s


def test_fmix32_vectors():
    for ln in read_golden("hash_vectors.txt"):
        a, b = ln.split()
        assert oracle.lib().orc_fmix32(int(a, 16)) == int(b, 16)
