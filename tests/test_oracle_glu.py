"""Pins of the oracle's gated-activation variants (clamped SwiGLU and SiTU-GLU).

The constants come from tests/golden/glu_variants.txt (cited there).  Each pin
is a limit, a bound or an identity that the pages' definitions fix, chosen so
that a plausible slip fails one of them:
- clamp: a lower clamp on the gate branch, a one-sided clamp on the up branch,
  or the clamp applied after SiLU;
- SiTU-GLU: beta * tanh(x) instead of beta * tanh(x / beta), the two betas
  swapped, the sigmoid taken of the capped gate, a missing sigmoid;
- both: the variant reaching the expert FFN and the whole layer (shared expert
  included), with the method's rounding point h = round(a).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


def _consts():
    c = {}
    for ln in read_golden("glu_variants.txt"):
        name, *vals = ln.split()
        c[name] = [float(v) for v in vals]
    return c


C = _consts()
GMAX, ULO, UHI = C["clamp"]
B1, B2, BOUND = C["situ"]


def silu_mul(g, u):  # SwiGLU itself is pinned in test_oracle_ffn_layer.py
    return oracle.glu_value(g, u, "swiglu")


GRID = [-1e4, -60.0, -12.0, -10.0, -3.0, -0.5, 0.0, 1e-3, 0.7, 4.0, 9.99, 10.0, 10.5, 37.0, 1e4]


def test_clamp_matches_swiglu_inside_the_box():
    for g in GRID:
        for u in GRID:
            if g <= GMAX and ULO <= u <= UHI:
                assert oracle.glu_value(g, u, "clamp") == silu_mul(g, u), (g, u)


def test_clamp_saturates_each_branch():
    for u in (-7.0, 0.3, 9.0):
        for g in (10.5, 37.0, 1e4):
            assert oracle.glu_value(g, u, "clamp") == silu_mul(GMAX, u)
    for g in (-3.0, 0.7, 9.0, 50.0):
        gg = min(g, GMAX)
        for u in (10.5, 1e4):
            assert oracle.glu_value(g, u, "clamp") == silu_mul(gg, UHI)
            assert oracle.glu_value(g, -u, "clamp") == silu_mul(gg, ULO)


def test_clamp_leaves_negative_gate_alone():
    # only max=10 on the gate: SiLU(-12) * u, not SiLU(-10) * u
    assert oracle.glu_value(-12.0, 2.0, "clamp") == silu_mul(-12.0, 2.0)
    assert oracle.glu_value(-12.0, 2.0, "clamp") != silu_mul(-10.0, 2.0)
    assert abs(oracle.glu_value(-60.0, 5.0, "clamp")) < 1e-20


def test_clamp_bound():
    top = silu_mul(GMAX, UHI)
    assert top == pytest.approx(GMAX * UHI, rel=1e-4)  # sigmoid(10) ~ 1 - 4.5e-5
    for g in GRID:
        for u in GRID:
            assert abs(oracle.glu_value(g, u, "clamp")) <= top


def test_situ_small_arguments_reduce_to_swiglu():
    # beta tanh(x / beta) = x (1 - (x/beta)^2 / 3 + ...): relative gap ~ 1e-8 here
    for g, u in ((1e-3, 2e-3), (-2e-3, 1e-3), (5e-4, -7e-4)):
        r = oracle.glu_value(g, u, "situ") / silu_mul(g, u)
        assert abs(r - 1.0) < 1e-7, (g, u, r)
    # ... and the caps are visible well before saturation
    assert oracle.glu_value(2.0, 2.0, "situ") < 0.95 * silu_mul(2.0, 2.0)


def test_situ_gate_branch_caps_at_beta_gate():
    # g -> inf: sigmoid -> 1, beta1 tanh(g/beta1) -> beta1; small u: up branch ~ u
    for u in (1e-3, -2e-3):
        assert oracle.glu_value(1e4, u, "situ") == pytest.approx(B1 * u, rel=1e-6)


def test_situ_up_branch_caps_at_beta_up():
    # u -> inf: up branch -> beta2; small g: gate branch ~ g sigmoid(g) = SiLU(g)
    for g in (1e-3, -2e-3):
        assert oracle.glu_value(g, 1e4, "situ") == pytest.approx(B2 * silu_mul(g, 1.0), rel=1e-6)
        assert oracle.glu_value(g, -1e4, "situ") == pytest.approx(-B2 * silu_mul(g, 1.0), rel=1e-6)


def test_situ_sigmoid_takes_the_uncapped_gate():
    # sigmoid(-60) ~ 1e-26: the product vanishes; sigmoid of the capped gate
    # (-4) would leave about -0.07 * up.
    assert abs(oracle.glu_value(-60.0, 20.0, "situ")) < 1e-20
    assert abs(oracle.glu_value(-1e4, 1e4, "situ")) == 0.0


def test_situ_product_bound():
    assert oracle.glu_value(1e4, 1e4, "situ") == BOUND
    assert oracle.glu_value(1e4, -1e4, "situ") == -BOUND
    for g in GRID:
        for u in GRID:
            assert abs(oracle.glu_value(g, u, "situ")) <= BOUND
    # the page's worked example: 20 x 30 = 600 without the caps, below 100 with them
    assert silu_mul(20.0, 30.0) == pytest.approx(600.0, abs=1e-3)
    assert 50.0 < oracle.glu_value(20.0, 30.0, "situ") < BOUND


@pytest.mark.parametrize("glu", ["swiglu", "clamp", "situ"])
def test_glu_odd_in_up_and_nan(glu):
    for g in GRID:
        for u in (0.3, 12.0, 40.0):
            assert oracle.glu_value(g, -u, glu) == -oracle.glu_value(g, u, glu)
    assert math.isnan(oracle.glu_value(float("nan"), 1.0, glu))
    assert math.isnan(oracle.glu_value(1.0, float("nan"), glu))


def bf16_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16(a):
    return synth.f32_to_bf16(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("glu", ["clamp", "situ"])
def test_expert_ffn_applies_the_variant(act, glu):
    # one-hot rows: h[r, i] = round(a(g_i, u_i)) with chosen branch values
    pairs = [(20.0, 30.0), (-12.0, 2.0), (11.0, -40.0), (0.5, 0.25), (6.0, 12.0)]
    I, D = len(pairs), 8
    x = np.zeros((1, D), np.float32)
    x[0, 0] = 1.0
    wg = np.zeros((I, D), np.float32)
    wu = np.zeros((I, D), np.float32)
    wd = np.zeros((D, I), np.float32)
    for i, (g, u) in enumerate(pairs):
        wg[i, 0], wu[i, 0] = g, u
    wd[0, 0] = 1.0
    if act == "bf16":
        x, wg, wu, wd = map(to_bf16, (x, wg, wu, wd))
    _, h = oracle.expert_ffn(x, wg, wu, wd, act, want_h=True, glu=glu)
    hv = h[0].astype(np.float64) if act == "f32" else bf16_to_f64(h[0])
    for i, (g, u) in enumerate(pairs):
        a = oracle.glu_value(g, u, glu)
        want = float(np.float32(a)) if act == "f32" else float(bf16_to_f64(
            oracle.bf16_from_f64_array(np.array([a]))[0]))
        assert hv[i] == want, (i, g, u, hv[i], want)


@pytest.mark.parametrize("glu", ["swiglu", "clamp", "situ"])
def test_layer_passes_the_variant_to_routed_and_shared(glu):
    # E=1, k=1, weight 1: y = round(o + s), where o and s are each the expert
    # FFN of the same variant; large weights drive the branches past the caps.
    rng = np.random.default_rng(11)
    T, D, I, Is = 6, 32, 16, 8
    x = to_bf16(rng.standard_normal((T, D)))
    m = tuple(to_bf16(3.0 * rng.standard_normal(s)) for s in ((I, D), (I, D), (D, I)))
    sh = tuple(to_bf16(3.0 * rng.standard_normal(s)) for s in ((Is, D), (Is, D), (D, Is)))
    wr = to_bf16(0.02 * rng.standard_normal((1, D)))
    y, idx, w, _ = oracle.layer_forward(x, None, wr, None, {0: m}, sh, T, D, 1, 1, I, Is,
                                        "softmax", "bf16", glu=glu)
    o = oracle.expert_ffn(x, *m, "bf16", glu=glu)
    s = oracle.expert_ffn(x, *sh, "bf16", glu=glu)
    ref = oracle.combine(o, idx, w, np.arange(T, dtype=np.int32), s, T, 1, D)
    assert np.array_equal(y, ref)
    if glu != "swiglu":
        plain = oracle.expert_ffn(x, *m, "bf16")
        assert not np.array_equal(plain, o)  # the caps were reached
