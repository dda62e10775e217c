"""Pins of the oracle's residual add + RMSNorm (the next block's input norm at
the end of the MoE tail).

- the page's worked example x = [3, 4] (tests/golden/rmsnorm_worked_example.txt);
- scale invariance RMSNorm(c u) = RMSNorm(u) (the page's 100x argument), exact
  for c = 64;
- the output's RMS is 1 with unit gain;
- the gain is per dimension: powers of two scale each output exactly;
- epsilon sits inside the square root, added to the mean of squares;
- the residual is added, and rounded to the activation type, before the norm.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


def bf16_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64(a):
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def cast(a, act):
    a = np.asarray(a, dtype=np.float32)
    return synth.f32_to_bf16(a) if act == "bf16" else a


def norm(x, act, gamma=None, res=None, eps=0.0):
    x = cast(x, act)
    T, D = x.shape
    res = cast(np.zeros((T, D)) if res is None else res, act)
    gamma = cast(np.ones(D) if gamma is None else gamma, act)
    return oracle.residual_rmsnorm(x, res, gamma, eps)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_worked_example(act):
    (lhs, rms_s, vals_s, tol_s), = [[p.strip() for p in ln.split("|")]
                                    for ln in read_golden("rmsnorm_worked_example.txt")]
    x = np.array([[float(v) for v in lhs.split()]])
    want = [float(v) for v in vals_s.split()]
    tol = float(tol_s)
    _, n = norm(x, act)
    got = f64(n)[0]
    step = 0.0 if act == "f32" else 2.0 ** -9  # bf16 output rounding (relative)
    for g, w in zip(got, want):
        assert abs(g - w) <= tol + step * abs(g), (got, want)
    if act == "f32":
        assert x[0, 0] / got[0] == pytest.approx(float(rms_s), abs=tol)
        assert np.sqrt(np.mean(got ** 2)) == pytest.approx(1.0, abs=1e-6)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_scale_invariance(act):
    u = synth.normal_f32(71, 0, 4 * 96, 1.0).reshape(4, 96)
    _, a = norm(u, act)
    _, b = norm(64.0 * u, act)  # power of two: the inputs scale exactly
    assert np.array_equal(a, b)
    if act == "f32":
        _, c = norm(100.0 * u, act)
        assert np.allclose(f64(c), f64(a), rtol=2e-6, atol=0)


def test_unit_gain_gives_unit_rms():
    u = synth.normal_f32(72, 0, 8 * 200, 3.0).reshape(8, 200)
    _, n = norm(u, "f32")
    rms = np.sqrt(np.mean(f64(n) ** 2, axis=1))
    assert np.allclose(rms, 1.0, atol=1e-6)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_gain_is_per_dimension(act):
    D = 64
    u = synth.normal_f32(73, 0, 3 * D, 1.0).reshape(3, D)
    g = 2.0 ** (np.arange(D) % 7 - 3)  # 1/8 .. 8, distinct per position
    _, n1 = norm(u, act)
    _, ng = norm(u, act, gamma=g)
    assert np.array_equal(f64(ng), f64(n1) * g[None, :])


def test_epsilon_inside_the_root():
    # h = [1, 1, 1, 1]: mean(h^2) = 1; eps = 3 gives RMS = sqrt(1 + 3) = 2 exactly
    _, n = norm(np.ones((1, 4)), "f32", eps=3.0)
    assert np.all(n == 0.5)
    # a zero row stays zero (no 0/0) with a positive epsilon
    _, z = norm(np.zeros((1, 8)), "f32", eps=1e-6)
    assert np.all(z == 0.0)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_residual_is_added_and_rounded_first(act):
    rng = np.random.default_rng(74)
    T, D = 5, 48
    x = cast(rng.standard_normal((T, D)), act)
    r = cast(rng.standard_normal((T, D)), act)
    g = cast(rng.uniform(0.5, 2.0, D), act)
    h, n = oracle.residual_rmsnorm(x, r, g, 1e-6)
    # the new residual is round(x + r) ...
    want_h = cast((f64(x) + f64(r)).astype(np.float32), act) if act == "f32" else \
        oracle.bf16_from_f64_array(f64(x) + f64(r))
    assert np.array_equal(h, want_h)
    # ... and the norm sees exactly that rounded value
    _, n2 = oracle.residual_rmsnorm(h, np.zeros_like(h), g, 1e-6)
    assert np.array_equal(n, n2)
    if act == "bf16":
        # bf16 steps by 2^-7 above 1: 1 + 2^-9 is below the midpoint and rounds
        # to 1, 1 + 3 * 2^-9 is above it and rounds up to 1 + 2^-7
        one = synth.f32_to_bf16(np.array([[1.0, 1.0]], np.float32))
        small = synth.f32_to_bf16(np.array([[2.0 ** -9, 3 * 2.0 ** -9]], np.float32))
        hh, _ = oracle.residual_rmsnorm(one, small, synth.f32_to_bf16(np.ones(2, np.float32)), 0.0)
        assert list(f64(hh)[0]) == [1.0, 1.0 + 2.0 ** -7]
