"""GPU routing and permutation vs the oracle: bit-exact indices, weights,
counts, offsets, rows (through the C-ABI)."""
import numpy as np
import pytest
import torch

import invariant_moe_amd as moe
import oracle
import synth
from gpu_util import banner, dev, requires_gpu, to_np

pytestmark = [pytest.mark.gpu, requires_gpu]


def _routing_case(cfg, T=None, offset=0):
    T = cfg.T if T is None else T
    x = synth.x_tokens(cfg, T=T, offset_tokens=offset)
    if cfg.route == "hash":
        ids = synth.token_ids(cfg, T=T, offset_tokens=offset)
        ref_idx, ref_w = oracle.route(None, None, ids, T, cfg.E, cfg.k, "hash")
        idx, w = moe.router_topk(None, None, None, dev(ids), cfg.E, cfg.k, "hash")
    else:
        wr = synth.router_weight(cfg)
        bias = synth.router_bias(cfg)
        logits = oracle.router_logits(x, wr)
        ref_idx, ref_w = oracle.route(logits, bias, None, T, cfg.E, cfg.k, cfg.route)
        idx, w = moe.router_topk(dev(x), dev(wr), None if bias is None else dev(bias), None,
                                 cfg.E, cfg.k, cfg.route)
    return to_np(idx), to_np(w), ref_idx, ref_w


@pytest.mark.parametrize("cid,T", [(1, None), (1, 3), (1, 10), (2, None), (2, 1), (2, 12),
                                   (2, 33), (4, 64), (4, 1), (4, 9), (5, None), (3, 300)])
def test_router_bitwise(cid, T):
    cfg = synth.CONFIGS[cid]
    banner(f"router cfg{cid} T={T}")
    idx, w, ref_idx, ref_w = _routing_case(cfg, T)
    assert np.array_equal(idx, ref_idx)
    assert np.array_equal(w.view(np.uint32), ref_w.view(np.uint32))


@pytest.mark.slow
def test_router_bitwise_full_prefill():
    banner("router cfg3 T=4096")
    idx, w, ref_idx, ref_w = _routing_case(synth.CONFIGS[3])
    assert np.array_equal(idx, ref_idx)
    assert np.array_equal(w.view(np.uint32), ref_w.view(np.uint32))


def _f32_stride(stride, start=0):
    bits = np.arange(start, 2**32, stride, dtype=np.uint64).astype(np.uint32)
    return bits.view(np.float32)


@pytest.mark.parametrize("mode", ["sigmoid", "softmax"])
def test_routing_scores_bitwise_sweep(mode):
    """Sigmoid keys / routing exp over a stride of all 2^32 fp32 bit patterns."""
    banner(f"routing scores sweep {mode}")
    x = _f32_stride(257, start=11)
    got = to_np(moe.routing_scores(dev(x), mode))
    ref = oracle.sigmoid_array(x) if mode == "sigmoid" else oracle.exp_array(x)
    gb, rb = got.view(np.uint32), ref.view(np.uint32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(gb[~nan], rb[~nan])


@pytest.mark.slow
def test_routing_sigmoid_exhaustive():
    """Every fp32 input: GPU sigmoid key == oracle sigmoid key, bitwise."""
    chunk = 1 << 28
    for c in range(16):
        banner(f"sigmoid exhaustive chunk {c}/16")
        bits = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        got = to_np(moe.routing_scores(dev(x), "sigmoid")).view(np.uint32)
        ref = oracle.sigmoid_array(x).view(np.uint32)
        nan = (ref & 0x7FFFFFFF) > 0x7F800000
        assert np.array_equal((got & 0x7FFFFFFF) > 0x7F800000, nan)
        assert np.array_equal(got[~nan], ref[~nan])


def test_router_ties_and_edges():
    banner("router ties / edges")
    # all-zero activations: every logit is +0 -> experts 0..k-1, weights 1/k
    T, D, E = 5, 256, 16
    x = np.zeros((T, D), np.uint16)
    wr = synth.normal_bf16(0, 0, E * D, 0.02).reshape(E, D)
    for mode in ("softmax", "sigmoid"):
        for k in (1, 4, 16):
            idx, w = moe.router_topk(dev(x), dev(wr), None, None, E, k, mode)
            assert np.array_equal(to_np(idx), np.tile(np.arange(k), (T, 1)))
            assert np.all(to_np(w) == np.float32(1.0 / k))
    # a huge bias sends every token to the same k experts (ties broken by id)
    x = synth.normal_bf16(1, 0, T * D, 1.0).reshape(T, D)
    bias = np.zeros(E, np.float32)
    bias[[3, 9]] = 100.0
    idx, w = moe.router_topk(dev(x), dev(wr), dev(bias), None, E, 2, "sigmoid")
    logits = oracle.router_logits(x, wr)
    ref_idx, ref_w = oracle.route(logits, bias, None, T, E, 2, "sigmoid")
    assert np.array_equal(to_np(idx), ref_idx)
    assert set(np.unique(ref_idx)) == {3, 9}
    assert np.array_equal(to_np(w).view(np.uint32), ref_w.view(np.uint32))
    # odd E (not a multiple of 64), k = E
    E2 = 29
    wr2 = synth.normal_bf16(2, 0, E2 * D, 0.05).reshape(E2, D)
    idx, w = moe.router_topk(dev(x), dev(wr2), None, None, E2, E2, "softmax")
    logits = oracle.router_logits(x, wr2)
    ref_idx, ref_w = oracle.route(logits, None, None, T, E2, E2, "softmax")
    assert np.array_equal(to_np(idx), ref_idx)
    assert np.array_equal(to_np(w).view(np.uint32), ref_w.view(np.uint32))


@pytest.mark.parametrize("T,E,k", [(9, 300, 8), (20, 1000, 32), (3, 1024, 1)])
@pytest.mark.parametrize("mode", ["softmax", "sigmoid"])
def test_router_many_experts_bitwise(T, E, k, mode):
    """Top-k over 8 and 16 keys per lane (E up to the 1024 limit, k up to 32),
    with and without a bias: indices and weights bit-exact."""
    banner(f"router E={E} k={k} {mode}")
    D = 256
    x = synth.normal_bf16(40, 0, T * D, 1.0).reshape(T, D)
    wr = synth.normal_bf16(41, 0, E * D, 0.05).reshape(E, D)
    logits = oracle.router_logits(x, wr)
    rng = np.random.default_rng(E + k)
    for bias in (None, (rng.standard_normal(E) * 0.01).astype(np.float32)):
        idx, w = moe.router_topk(dev(x), dev(wr), None if bias is None else dev(bias), None, E, k,
                                 mode)
        ref_idx, ref_w = oracle.route(logits, bias, None, T, E, k, mode)
        assert np.array_equal(to_np(idx), ref_idx)
        assert np.array_equal(to_np(w).view(np.uint32), ref_w.view(np.uint32))


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (64, 64, 6), (65, 64, 6), (300, 256, 8),
                                   (4096, 256, 8), (1000, 1024, 32), (7, 3, 3), (130, 1, 1)])
def test_permute_bitwise(T, E, k):
    banner(f"permute T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 1000 + E)
    # skewed choice of experts, distinct per token
    p = rng.dirichlet(np.ones(E) * 0.3)
    idx = np.array([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)],
                   dtype=np.int32).reshape(T, k)
    counts, offsets, row_token, pair_row, _ = moe.permute(dev(idx), E)
    rc, ro, rt, rp = oracle.permute(idx, E)
    assert np.array_equal(to_np(counts), rc)
    assert np.array_equal(to_np(offsets), ro)
    assert np.array_equal(to_np(row_token), rt)
    assert np.array_equal(to_np(pair_row), rp)


def test_permute_gather():
    banner("permute gather")
    cfg = synth.CONFIGS[2].with_T(100)
    x = synth.x_tokens(cfg)
    rng = np.random.default_rng(5)
    idx = np.array([rng.permutation(cfg.E)[:cfg.k] for _ in range(cfg.T)], dtype=np.int32)
    _, _, row_token, _, x_perm = moe.permute(dev(idx), cfg.E, x=dev(x))
    rt = oracle.permute(idx, cfg.E)[2]
    assert np.array_equal(to_np(x_perm), x[rt])


def test_hash_routing_edges():
    banner("hash edges")
    ids = np.array([0, 1, 131071, 5, 5, 77], dtype=np.int32)
    for E, k in [(1, 1), (7, 7), (256, 8), (1024, 32), (3, 2)]:
        idx, w = moe.router_topk(None, None, None, dev(ids), E, k, "hash")
        ref_idx, ref_w = oracle.route(None, None, ids, len(ids), E, k, "hash")
        assert np.array_equal(to_np(idx), ref_idx)
        assert np.array_equal(to_np(w).view(np.uint32), ref_w.view(np.uint32))


def test_softmax_bias_reorders_experts():
    """Softmax routing where a bias ranks small logits first: the weights shift
    by the largest selected logit (finite), bit-equal to the oracle.  Logits are
    exact: x = e_0, W_r[e, 0] = the wanted logit (bf16-exact values)."""
    banner("softmax with a reordering bias")
    E, D, k, T = 64, 64, 4, 5
    rng = np.random.default_rng(11)
    lv = np.round(rng.uniform(-120, 120, size=(T, E))).astype(np.float32)
    # token t: its own router row block -> use one W_r and per-token x = e_t
    wr = np.zeros((E, D), np.float32)
    x = np.zeros((T, D), np.float32)
    for t in range(T):
        x[t, t] = 1.0
        wr[:, t] = lv[t]
    bias = np.zeros(E, np.float32)
    bias[:8] = 1000.0  # experts 0..7 always selected, whatever their logits
    xb, wb = synth.f32_to_bf16(x), synth.f32_to_bf16(wr)
    logits = oracle.router_logits(xb, wb)
    assert np.array_equal(logits, lv)
    ref_idx, ref_w = oracle.route(logits, bias, None, T, E, k, "softmax")
    assert np.all(np.isfinite(ref_w))
    idx, w = moe.router_topk(dev(xb), dev(wb), dev(bias), None, E, k, "softmax")
    assert np.array_equal(to_np(idx), ref_idx)
    assert np.array_equal(to_np(w).view(np.uint32), ref_w.view(np.uint32))
