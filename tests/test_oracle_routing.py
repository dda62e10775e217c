"""Pins of the oracle's routing and dispatch.

- logit order: hand-derived golden cases (tests/golden/router_order.txt);
- logit value: within the recursive-summation error bound of the exact dot
  product (Fractions);
- top-k: brute force with Python's sort on (key desc, id asc); constructed ties;
- weights: normalise to 1 (sum within k*2^-23) and equal the full softmax
  renormalised over the selected experts (the same quantity in exact arithmetic);
- hash routing: k=1 is fmix32(token_id) mod E (DeepSeek-V4 infra walkthrough,
  section 6.3: expert = hash(token id) mod number of experts), fmix32 pinned by
  its published vectors; slots distinct; uniform load;
- permutation: Python's stable sort of (expert, token) pairs.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import read_golden


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(a, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "value is not exact in bf16"
    return (b >> 16).astype(np.uint16)


def test_router_order_golden():
    cases = read_golden("router_order.txt")
    assert len(cases) >= 5
    for ln in cases:
        lhs, rhs = ln.split("=")
        toks = lhs.split()
        acts, D, items = toks[0].split(","), int(toks[1]), toks[2:]
        x = np.zeros((1, D), dtype=np.float32)
        w = np.zeros((1, D), dtype=np.float32)
        for it in items:
            d, xv, wv = it.split(":")
            x[0, int(d)] = float.fromhex(xv) if "0x" in xv else float(xv)
            w[0, int(d)] = float.fromhex(wv) if "0x" in wv else float(wv)
        want = float.fromhex(rhs.strip())
        for act in acts:
            if act == "f32":
                got = oracle.router_logits(x, w)
            else:
                got = oracle.router_logits(_bf16_bits(x), _bf16_bits(w))
            assert got[0, 0] == np.float32(want), (ln, act, got[0, 0])


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_router_logit_error_bound(act):
    rng = np.random.default_rng(1)
    T, E, D = 3, 4, 512
    x = rng.standard_normal((T, D)).astype(np.float32)
    w = (0.02 * rng.standard_normal((E, D))).astype(np.float32)
    if act == "bf16":
        x = (_round_bf16(x))
        w = (_round_bf16(w))
        xa, wa = _bf16_bits(x), _bf16_bits(w)
    else:
        xa, wa = x, w
    got = oracle.router_logits(xa, wa)
    u = 2.0**-24
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], w[e]))
            mag = float(np.sum(np.abs(x[t].astype(np.float64) * w[e])))
            # each value passes through at most D/64/8*8 + 6 roundings
            n = D // 64 + 6
            bound = (n * u / (1 - n * u)) * mag
            assert abs(Fraction(float(got[t, e])) - exact) <= Fraction(bound)


def _round_bf16(a):
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _brute_topk(keys, k):
    order = sorted(range(len(keys)), key=lambda e: (-float(keys[e]), e))
    return order[:k]


@pytest.mark.parametrize("mode", ["softmax", "sigmoid"])
def test_topk_brute_force(mode):
    rng = np.random.default_rng(2)
    for trial in range(30):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, E + 1))
        T = 5
        # coarse logits so ties are frequent
        logits = (rng.integers(-4, 5, size=(T, E)) * 0.25).astype(np.float32)
        bias = (rng.integers(-2, 3, size=E) * 0.125).astype(np.float32) if trial % 2 else None
        idx, w, keys = oracle.route(logits, bias, None, T, E, k, mode, want_keys=True)
        for t in range(T):
            assert list(idx[t]) == _brute_topk(keys[t], k)
            s = logits[t] if mode == "softmax" else 1 / (1 + np.exp(-logits[t].astype(np.float64)))
            if bias is None:
                assert np.allclose(keys[t], s, rtol=1e-6, atol=1e-7)
            else:
                assert np.allclose(keys[t], s + bias, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("mode", ["softmax", "sigmoid"])
@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_all_ties_pick_lowest_ids_and_uniform_weights(mode, k):
    E, T = 16, 3
    logits = np.zeros((T, E), dtype=np.float32)
    logits[1] = -0.0  # +0 and -0 compare equal
    idx, w = oracle.route(logits, None, None, T, E, k, mode)
    assert np.array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.all(w == np.float32(1.0 / k))  # exact for power-of-two k


def test_bias_decides_selection_not_weights():
    E, k = 8, 2
    logits = np.array([[0.1, 0.2, 0.3, 0.4, 0.5, 0.6, 0.7, 0.8]], dtype=np.float32)
    bias = np.zeros(E, dtype=np.float32)
    bias[0] = bias[1] = 10.0
    idx, w, keys = oracle.route(logits, bias, None, 1, E, k, "sigmoid", want_keys=True)
    assert list(idx[0]) == [1, 0]  # sigmoid(0.2)+10 > sigmoid(0.1)+10
    s = 1 / (1 + np.exp(-np.array([0.2, 0.1])))
    assert np.allclose(w[0], s / s.sum(), rtol=1e-6)


@pytest.mark.parametrize("mode", ["softmax", "sigmoid"])
def test_weights_normalise_and_match_full_softmax(mode):
    rng = np.random.default_rng(3)
    T, E, k = 200, 64, 6
    logits = (1.7 * rng.standard_normal((T, E))).astype(np.float32)
    idx, w = oracle.route(logits, None, None, T, E, k, mode)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0**-23)
    l64 = logits.astype(np.float64)
    for t in range(T):
        sel = idx[t]
        if mode == "softmax":
            full = np.exp(l64[t] - l64[t].max())
            full /= full.sum()
            ref = full[sel] / full[sel].sum()  # renormalised full softmax
        else:
            s = 1 / (1 + np.exp(-l64[t]))
            ref = s[sel] / s[sel].sum()
        assert np.allclose(w[t], ref, rtol=2e-6, atol=1e-9)


def test_hash_routing_k1_closed_form():
    fmix = oracle.lib().orc_fmix32
    ids = np.array([0, 1, 2, 7, 131071, 65536, 12345], dtype=np.int32)
    for E in (1, 7, 64, 256):
        idx, w = oracle.route(None, None, ids, len(ids), E, 1, "hash")
        for t, tid in enumerate(ids):
            assert idx[t, 0] == fmix(int(tid)) % E
            assert w[t, 0] == 1.0


def test_hash_routing_slots_distinct_uniform():
    T, E, k = 131072, 256, 8
    ids = np.arange(T, dtype=np.int32)
    idx, w = oracle.route(None, None, ids, T, E, k, "hash")
    s = np.sort(idx, axis=1)
    assert np.all(np.diff(s, axis=1) > 0)
    assert np.all(w == np.float32(0.125))
    counts = np.bincount(idx.ravel(), minlength=E)
    expect = T * k / E
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    # chi-square with 255 dof: mean 255, sd ~22.6; 400 is > 6 sd
    assert chi2 < 400, chi2
    # k = E: every expert exactly once per token
    idx2, _ = oracle.route(None, None, ids[:100], 100, 5, 5, "hash")
    assert np.all(np.sort(idx2, axis=1) == np.arange(5))


def test_permute_is_stable_counting_sort():
    rng = np.random.default_rng(4)
    for T, E, k in [(1, 4, 2), (37, 8, 3), (300, 64, 6), (5, 1, 1), (0, 3, 2)]:
        idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
        counts, offsets, row_token, pair_row = oracle.permute(idx, E)
        pairs = sorted(((int(idx[t, j]), t, j) for t in range(T) for j in range(k)),
                       key=lambda p: p[0])  # Python's sort is stable
        assert [t for _, t, _ in pairs] == list(row_token)
        for r, (e, t, j) in enumerate(pairs):
            assert pair_row[t * k + j] == r
        assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
        assert offsets[0] == 0 and offsets[E] == T * k
        assert np.array_equal(np.diff(offsets), counts)


def test_hash_slots_from_published_fmix32_values():
    """Slot j of token tid hashes tid + j * 0x9E3779B9; for the token ids of
    tests/golden/hash_slots.txt that argument is an input whose fmix32 value is
    published, so the slot's expert is known without the oracle's hash."""
    cases = read_golden("hash_slots.txt")
    assert len(cases) >= 6
    for ln in cases:
        tid, E, k, j, inp, want = ln.split()
        tid_u, E, k, j, want = int(tid, 16), int(E), int(k), int(j), int(want)
        assert (tid_u + j * 0x9E3779B9) % (1 << 32) == int(inp, 16)
        ids = np.array([tid_u], dtype=np.uint32).view(np.int32)
        idx, w = oracle.route(None, None, ids, 1, E, k, "hash")
        assert want not in list(idx[0, :j]), ln  # no earlier slot took it: no probing
        assert idx[0, j] == want, (ln, idx[0])
        assert np.all(w == np.float32(1.0 / k))


def test_softmax_shift_is_the_largest_selected_logit():
    """A bias can rank an expert with a small logit first; the weights must
    still be the renormalised softmax over the selected logits (finite, summing
    to 1).  Shifting by the rank-0 logit would give exp(100) = inf here."""
    E, k = 6, 3
    logits = np.array([[0.0, 100.0, 99.0, -5.0, 3.0, 1.0]], dtype=np.float32)
    bias = np.zeros(E, dtype=np.float32)
    bias[0] = 1000.0  # expert 0 (logit 0) ranks first
    idx, w = oracle.route(logits, bias, None, 1, E, k, "softmax")
    assert list(idx[0]) == [0, 1, 2]
    assert np.all(np.isfinite(w))
    sel = logits[0, idx[0]].astype(np.float64)
    ref = np.exp(sel - sel.max())
    ref /= ref.sum()
    assert np.allclose(w[0], ref, rtol=2e-6, atol=1e-30)
    assert abs(float(w[0].astype(np.float64).sum()) - 1.0) <= k * 2.0**-23
    # without a bias the shift is the rank-0 logit, as before
    idx2, w2 = oracle.route(logits, None, None, 1, E, k, "softmax")
    assert list(idx2[0]) == [1, 2, 4]
    ref2 = np.exp(logits[0, [1, 2, 4]].astype(np.float64) - 100.0)
    assert np.allclose(w2[0], ref2 / ref2.sum(), rtol=2e-6)
