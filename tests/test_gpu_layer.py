"""GPU expert FFN, combine and whole layer vs the oracle (through the C-ABI).

Stage parity follows the isolation method of the Fireworks parity post
(swap one block for the reference): each GPU stage is fed the oracle's output
of the previous stage.  End to end: indices bit-exact and rel-L2 of y within
1e-5 (fp32) / 2e-3 (bf16, MXFP4).  At the full prefill sizes the oracle
computes a sample of tokens (a token's output depends only on that token).
"""
import numpy as np
import pytest
import torch

import invariant_moe_amd as moe
import oracle
import synth
from gpu_util import banner, dev, device_layer, rel_l2, requires_gpu, to_np, tol_for
from gpu_util import mxfp4_decode_bf16 as _decode_bf16, mxfp4_pack as _pack
from synth import device as sdev

pytestmark = [pytest.mark.gpu, requires_gpu]


def _oracle_layer(cfg, x, ids, experts=None):
    if experts is None:
        experts = {e: synth.expert_matrices(cfg, e) for e in range(cfg.E)}
    return oracle.layer_forward(x, ids, synth.router_weight(cfg) if cfg.route != "hash" else None,
                                synth.router_bias(cfg), experts, synth.shared_matrices(cfg),
                                x.shape[0], cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.route,
                                cfg.wdtype)


def _device_layer(cid):
    return device_layer(cid)


@pytest.mark.parametrize("cid", [1, 2])
def test_layer_full_vs_oracle(cid):
    cfg = synth.CONFIGS[cid]
    banner(f"layer cfg{cid} full T={cfg.T}")
    dl, layer = _device_layer(cid)
    x = synth.x_tokens(cfg)
    y = to_np(layer.forward(dev(x)))
    y_ref, idx_ref, w_ref, _ = _oracle_layer(cfg, x, None)
    r = rel_l2(y, y_ref)
    banner(f"cfg{cid} rel_l2={r:.3e}")
    assert r <= tol_for(cfg.act)


def test_stage_parity_swap_in():
    """Each GPU stage from the oracle's previous-stage output (recipe 2)."""
    cfg = synth.CONFIGS[2].with_T(200)
    banner("stage parity recipe 2, T=200")
    x = synth.x_tokens(cfg)
    wr, bias = synth.router_weight(cfg), synth.router_bias(cfg)
    logits = oracle.router_logits(x, wr)
    idx, w = oracle.route(logits, bias, None, cfg.T, cfg.E, cfg.k, cfg.route)
    counts, offsets, row_token, pair_row = oracle.permute(idx, cfg.E)
    ex = {e: synth.expert_matrices(cfg, e) for e in range(cfg.E)}
    # oracle expert outputs per expert group
    o_ref = np.empty((cfg.T * cfg.k, cfg.D), np.uint16)
    for e in range(cfg.E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            o_ref[a:b] = oracle.expert_ffn(np.ascontiguousarray(x[row_token[a:b]]), *ex[e], "bf16")
    sh = synth.shared_matrices(cfg)
    s_ref = oracle.expert_ffn(x, *sh, "bf16")
    y_ref = oracle.combine(o_ref, idx, w, pair_row, s_ref, cfg.T, cfg.k, cfg.D)
    # grouped GEMM stage (rows gathered through row_token) vs oracle
    dl, _ = _device_layer(2)
    routed = moe.ExpertWeights(dl.gate, dl.up, dl.down)
    o_gpu = to_np(moe.grouped_swiglu(dev(x), dev(row_token), dev(offsets), cfg.T * cfg.k, cfg.E,
                                     routed))
    r_o = rel_l2(o_gpu, o_ref)
    banner(f"grouped GEMM rel_l2={r_o:.3e}")
    assert r_o <= 2e-3
    shared = moe.ExpertWeights(dl.sh_gate, dl.sh_up, dl.sh_down)
    s_gpu = to_np(moe.grouped_swiglu(dev(x), None, dev(np.array([0, cfg.T], np.int32)), cfg.T, 1,
                                     shared))
    assert rel_l2(s_gpu, s_ref) <= 2e-3
    # combine stage on the oracle's o and s: bit-exact
    y_gpu = to_np(moe.combine(dev(o_ref), dev(idx), dev(w), dev(pair_row), dev(s_ref)))
    assert np.array_equal(y_gpu, y_ref)
    # combine without a shared expert
    y2 = to_np(moe.combine(dev(o_ref), dev(idx), dev(w), dev(pair_row), None))
    assert np.array_equal(y2, oracle.combine(o_ref, idx, w, pair_row, None, cfg.T, cfg.k, cfg.D))


def test_fp32_stage_parity():
    cfg = synth.CONFIGS[1]
    banner("fp32 stages recipe 1")
    x = synth.x_tokens(cfg)
    wr = synth.router_weight(cfg)
    idx, w = oracle.route(oracle.router_logits(x, wr), None, None, cfg.T, cfg.E, cfg.k, "softmax")
    counts, offsets, row_token, pair_row = oracle.permute(idx, cfg.E)
    ex = {e: synth.expert_matrices(cfg, e) for e in range(cfg.E)}
    o_ref = np.empty((cfg.T * cfg.k, cfg.D), np.float32)
    for e in range(cfg.E):
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            o_ref[a:b] = oracle.expert_ffn(np.ascontiguousarray(x[row_token[a:b]]), *ex[e], "f32")
    dl, _ = _device_layer(1)
    routed = moe.ExpertWeights(dl.gate, dl.up, dl.down)
    o_gpu = to_np(moe.grouped_swiglu(dev(x), dev(row_token), dev(offsets), cfg.T * cfg.k, cfg.E,
                                     routed))
    assert rel_l2(o_gpu, o_ref) <= 1e-5
    y_gpu = to_np(moe.combine(dev(o_ref), dev(idx), dev(w), dev(pair_row), None))
    assert np.array_equal(y_gpu.view(np.uint32),
                          oracle.combine(o_ref, idx, w, pair_row, None, cfg.T, cfg.k, cfg.D).view(np.uint32))


def test_grouped_gemm_past_owner_map():
    """More than 8192 row tiles (1.1 M rows in 128-row tiles): the tile tables
    find each tile's expert by binary search instead of the LDS owner map.
    Sampled rows match the oracle; the first rows match a small run bitwise."""
    banner("grouped GEMM, 1.1 M rows")
    E, D, I = 3, 64, 32
    sizes = np.array([400_000, 1, 700_123], dtype=np.int64)
    R = int(sizes.sum())
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rng = np.random.default_rng(51)
    x = synth.normal_bf16(52, 0, R * D, 1.0).reshape(R, D)
    mats = [synth.normal_bf16(53 + i, 0, E * r * c, 0.1).reshape(E, r, c)
            for i, (r, c) in enumerate(((I, D), (I, D), (D, I)))]
    w = moe.ExpertWeights(*(dev(m) for m in mats))
    out = to_np(moe.grouped_swiglu(dev(x), None, dev(offsets), R, E, w))
    rows = np.sort(np.concatenate([rng.choice(R, 300, replace=False), [0, R - 1, 400_000]]))
    for e in range(E):
        sel = rows[(rows >= offsets[e]) & (rows < offsets[e + 1])]
        if len(sel):
            ref = oracle.expert_ffn(np.ascontiguousarray(x[sel]), mats[0][e], mats[1][e],
                                    mats[2][e], "bf16")
            assert rel_l2(out[sel], ref) <= 2e-3, e
    small = to_np(moe.grouped_swiglu(dev(np.ascontiguousarray(x[:1000])), None,
                                     dev(np.array([0, 1000, 1000, 1000], np.int32)), 1000, E, w))
    assert np.array_equal(small, out[:1000])


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_combine_many_slots_bitwise(act):
    """Combine with k = 9, 17 and 32 slots (several batches of eight rows,
    clamped tail slots), ragged T, two row widths, with and without a shared
    expert: bit-exact against the oracle's fixed-order combine."""
    banner(f"combine many slots {act}")
    rng = np.random.default_rng(31)
    E = 40
    for T, k, D in ((37, 9, 256), (5, 17, 1056), (3, 32, 1056)):
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        w = rng.random((T, k), dtype=np.float32)
        _, _, _, pair_row = oracle.permute(idx, E)
        if act == "bf16":
            o = synth.normal_bf16(32, 0, T * k * D, 1.0).reshape(T * k, D)
            sh = synth.normal_bf16(33, 0, T * D, 1.0).reshape(T, D)
        else:
            o = rng.standard_normal((T * k, D), dtype=np.float32)
            sh = rng.standard_normal((T, D), dtype=np.float32)
        for shared in (sh, None):
            y = to_np(moe.combine(dev(o), dev(idx), dev(w), dev(pair_row),
                                  None if shared is None else dev(shared)))
            ref = oracle.combine(o, idx, w, pair_row, shared, T, k, D)
            assert np.array_equal(y.view(np.uint8), ref.view(np.uint8)), (T, k, D, shared is None)


def test_batch_invariance_small_layer():
    """Every token's output row is bitwise identical for batch sizes 1..64, for
    shuffled batches, and inside the full 512-token batch (recipe 2 weights;
    different T select different GEMM tile shapes)."""
    cfg = synth.CONFIGS[2]
    banner("batch invariance recipe 2")
    dl, layer = _device_layer(2)
    pool = synth.x_tokens(cfg)  # 512 tokens
    y_full = to_np(layer.forward(dev(pool)))
    rng = np.random.default_rng(0)
    for T in list(range(1, 65)) + [100, 257]:
        sel = np.arange(T)
        y = to_np(layer.forward(dev(np.ascontiguousarray(pool[sel]))))
        assert np.array_equal(y, y_full[sel]), T
        if T in (7, 64, 257):
            for _ in range(3):
                perm = rng.permutation(cfg.T)[:T]
                y = to_np(layer.forward(dev(np.ascontiguousarray(pool[perm]))))
                assert np.array_equal(y, y_full[perm]), ("shuffle", T)


def test_determinism_repeat_and_streams():
    cfg = synth.CONFIGS[2]
    banner("determinism")
    dl, layer = _device_layer(2)
    x = dev(synth.x_tokens(cfg))
    a = to_np(layer.forward(x))
    b = to_np(layer.forward(x))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = layer.forward(x, stream=s)
    s.synchronize()
    assert np.array_equal(a, b) and np.array_equal(a, to_np(c))


def test_side_streams_not_current():
    """forward on streams that are not the current one: each stream gets its
    own workspace and its outputs are allocated on it, so two calls in flight
    on two streams do not share memory; results equal the current stream's."""
    cfg = synth.CONFIGS[2]
    banner("side streams")
    dl, _ = _device_layer(2)
    layer = sdev.layer_object(dl)
    xa = dev(synth.x_tokens(cfg, T=300))
    xb = dev(synth.x_tokens(cfg, T=200, offset_tokens=300))
    ya, yb = to_np(layer.forward(xa)), to_np(layer.forward(xb))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):  # interleaved, no synchronisation between the streams
        outs.append((layer.forward(xa, stream=s1), layer.forward(xb, stream=s2)))
    s1.synchronize()
    s2.synchronize()
    assert len(layer._ws) >= 3  # current stream, s1, s2
    for a, b in outs:
        assert np.array_equal(to_np(a), ya) and np.array_equal(to_np(b), yb)
    # the plain entry points on a side stream
    idx, w = moe.router_topk(xa, dl.w_router, dl.bias, None, cfg.E, cfg.k, "sigmoid", stream=s1)
    s1.synchronize()
    ridx, rw = moe.router_topk(xa, dl.w_router, dl.bias, None, cfg.E, cfg.k, "sigmoid")
    assert torch.equal(idx, ridx) and torch.equal(w, rw)


def test_mxfp4_equals_bf16_on_decoded_weights():
    """MXFP4 expert weights through the grouped GEMM give the same bits as the
    bf16 path on the oracle-decoded weights (random codes, all 16 present)."""
    banner("mxfp4 vs bf16")
    E, I, D, T = 3, 64, 256, 40
    rng = np.random.default_rng(11)
    mats, dec = [], []
    for shape in ((E, I, D), (E, I, D), (E, D, I)):
        codes = rng.integers(0, 16, size=shape, dtype=np.uint8)
        scales = rng.integers(118, 124, size=(shape[0], shape[1], shape[2] // 32), dtype=np.uint8)
        packed = _pack(codes)
        mats.append((packed, scales))
        dec.append(_decode_bf16(packed, scales))
    x = synth.normal_bf16(9, 0, T * D, 1.0).reshape(T, D)
    idx = np.array([rng.permutation(E)[:2] for _ in range(T)], dtype=np.int32)
    _, offsets, row_token, _ = oracle.permute(idx, E)
    R = T * 2
    w4 = moe.ExpertWeights(dev(mats[0][0]), dev(mats[1][0]), dev(mats[2][0]),
                           dev(mats[0][1]), dev(mats[1][1]), dev(mats[2][1]))
    w16 = moe.ExpertWeights(dev(dec[0]), dev(dec[1]), dev(dec[2]))
    o4 = to_np(moe.grouped_swiglu(dev(x), dev(row_token), dev(offsets), R, E, w4))
    o16 = to_np(moe.grouped_swiglu(dev(x), dev(row_token), dev(offsets), R, E, w16))
    assert np.array_equal(o4, o16)
    ref = np.empty_like(o16)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        ref[a:b] = oracle.expert_ffn(np.ascontiguousarray(x[row_token[a:b]]), dec[0][e], dec[1][e],
                                     dec[2][e], "bf16")
    assert rel_l2(o4, ref) <= 2e-3


def test_mxfp4_scale_decode_exhaustive():
    """Every E2M1 code with every scale byte 0..252, decoded in the kernel, equals
    the oracle's exact value.  Token t is one-hot at d = 32 t (scale block t);
    gate = 1.0, down selects feature n % 32, so o[t, n] = round(silu(1) *
    up[n % 32, 32 t]) reads one decoded up-weight per output."""
    banner("mxfp4 decode exhaustive")
    NB = 253
    D, I, E = 32 * NB, 32, 1
    up_codes = np.broadcast_to((np.arange(I) % 16).astype(np.uint8)[:, None], (I, D))[None].copy()
    up_scales = np.broadcast_to(np.arange(NB, dtype=np.uint8)[None, :], (I, NB))[None].copy()
    gate_codes = np.full((1, I, D), 2, np.uint8)        # 1.0
    gate_scales = np.full((1, I, NB), 127, np.uint8)
    dn_codes = np.zeros((1, D, I), np.uint8)
    dn_codes[0, np.arange(D), np.arange(D) % I] = 2     # selector: 1.0 at i = n % 32
    dn_scales = np.full((1, D, 1), 127, np.uint8)
    mats = [(_pack(gate_codes), gate_scales), (_pack(up_codes), up_scales),
            (_pack(dn_codes), dn_scales)]
    dec = [_decode_bf16(p, s) for p, s in mats]
    w4 = moe.ExpertWeights(*(dev(m[0]) for m in mats), *(dev(m[1]) for m in mats))
    w16 = moe.ExpertWeights(*(dev(d) for d in dec))
    T = NB
    x = np.zeros((T, D), np.uint16)
    x[np.arange(T), 32 * np.arange(T)] = 0x3F80        # 1.0
    off = dev(np.array([0, T], np.int32))
    o4 = to_np(moe.grouped_swiglu(dev(x), None, off, T, E, w4))
    o16 = to_np(moe.grouped_swiglu(dev(x), None, off, T, E, w16))
    assert np.array_equal(o4, o16)
    # distinct codes give distinct outputs (the readout is not saturated)
    row = o16[NB // 2, :16]
    assert len(set(row[1:8].tolist())) == 7


def _rand_mxfp4(rng, shape):
    codes = rng.integers(0, 16, size=shape, dtype=np.uint8)
    scales = rng.integers(118, 124, size=(shape[0], shape[1], shape[2] // 32), dtype=np.uint8)
    packed = _pack(codes)
    return packed, scales, _decode_bf16(packed, scales)


def test_tile_brackets_and_weight_formats_bitwise():
    """Every row-tile bracket of the planner (<= 2, <= 16, <= 96 and more rows
    per expert) with MXFP4 routed experts next to a bf16 shared expert, the
    reverse, and both MXFP4: each layer gives the bits of the all-bf16 layer
    on the decoded weights, and a token's row is the same at every T."""
    banner("tile brackets x weight formats")
    E, k, D, I, Is = 4, 2, 288, 96, 64  # K % 64 == 32 in both GEMMs (trailing half step)
    rng = np.random.default_rng(23)
    routed = [_rand_mxfp4(rng, s) for s in ((E, I, D), (E, I, D), (E, D, I))]
    shared = [_rand_mxfp4(rng, s) for s in ((1, Is, D), (1, Is, D), (1, D, Is))]

    def fp4(m):
        return moe.ExpertWeights(*(dev(a[0]) for a in m), *(dev(a[1]) for a in m))

    def bf16(m):
        return moe.ExpertWeights(*(dev(a[2]) for a in m))

    w_router = dev(synth.normal_bf16(24, 0, E * D, 0.05).reshape(E, D))
    layers = {
        "bf16": moe.MoELayer(w_router, None, bf16(routed), bf16(shared), E, k, "softmax"),
        "routed mxfp4": moe.MoELayer(w_router, None, fp4(routed), bf16(shared), E, k, "softmax"),
        "shared mxfp4": moe.MoELayer(w_router, None, bf16(routed), fp4(shared), E, k, "softmax"),
        "both mxfp4": moe.MoELayer(w_router, None, fp4(routed), fp4(shared), E, k, "softmax"),
    }
    xs = synth.normal_bf16(25, 0, 600 * D, 1.0).reshape(600, D)
    y_all = None
    for T in (600, 150, 20, 3, 1):  # rows per expert T*k/E = 300, 75, 10, 1.5, 0.5
        x = dev(np.ascontiguousarray(xs[:T]))
        ys = {name: to_np(layer.forward(x)) for name, layer in layers.items()}
        for name, y in ys.items():
            assert np.array_equal(y, ys["bf16"]), (T, name)
        if y_all is None:
            y_all = ys["bf16"]
            assert ((y_all & 0x7F80) != 0x7F80).all()  # finite bf16
            assert np.count_nonzero(y_all & 0x7FFF) > y_all.size // 2
        else:
            assert np.array_equal(ys["bf16"], y_all[:T]), T


def test_layer_w4a8_full_size_sampled():
    """Recipe 5 at full size with MOE_FLAG_W4A8 (the launch configuration of
    bench.py --config 5 --w4a8); the oracle recomputes a sample of tokens
    stage by stage: hash routing, the FP4 x FP8 routed experts, the bf16 shared
    expert, the combine."""
    cfg = synth.CONFIGS[5]
    banner(f"layer cfg5 W4A8 full T={cfg.T} (sampled oracle)")
    dl, _ = _device_layer(5)
    layer = sdev.layer_object(dl, w4a8=True)
    x = synth.x_tokens(cfg)
    ids = synth.token_ids(cfg)
    y = to_np(layer.forward(dev(x), dev(ids)))
    rng = np.random.default_rng(55)
    sample = np.sort(rng.choice(cfg.T, size=3, replace=False))  # ~24 experts, ~2 s each
    sample[-1] = cfg.T - 1  # the ragged end
    n = len(sample)
    xs, ids_s = np.ascontiguousarray(x[sample]), np.ascontiguousarray(ids[sample])
    idx_s, w_s = oracle.route(None, None, ids_s, n, cfg.E, cfg.k, "hash")
    _, offs, row_tok, pair_row = oracle.permute(idx_s, cfg.E)
    o = np.empty((n * cfg.k, cfg.D), np.uint16)
    for e in np.unique(idx_s):
        a, b = offs[e], offs[e + 1]
        o[a:b] = oracle.expert_ffn_w4a8(np.ascontiguousarray(xs[row_tok[a:b]]),
                                        *synth.expert_matrices(cfg, int(e)))
    s = oracle.expert_ffn(xs, *synth.shared_matrices(cfg), "bf16")
    y_ref = oracle.combine(o, idx_s, w_s, pair_row, s, n, cfg.k, cfg.D)
    r = rel_l2(y[sample], y_ref)
    banner(f"cfg5 W4A8 sampled rel_l2={r:.3e}")
    assert r <= 2e-3


@pytest.mark.parametrize("cid,ntok", [(5, 12), (3, 12)])
def test_layer_full_size_sampled(cid, ntok):
    """Full-size batch on the GPU; the oracle recomputes a sample of tokens."""
    cfg = synth.CONFIGS[cid]
    banner(f"layer cfg{cid} full T={cfg.T} (sampled oracle)")
    dl, layer = _device_layer(cid)
    x = synth.x_tokens(cfg)
    ids = synth.token_ids(cfg) if cfg.route == "hash" else None
    y = to_np(layer.forward(dev(x), None if ids is None else dev(ids)))
    rng = np.random.default_rng(cid)
    sample = np.sort(rng.choice(cfg.T, size=ntok, replace=False))
    sample[0] = cfg.T - 1  # include the ragged end
    xs = np.ascontiguousarray(x[sample])
    ids_s = None if ids is None else np.ascontiguousarray(ids[sample])
    # route the sample with the oracle to know which experts it needs
    if cfg.route == "hash":
        idx_s, _ = oracle.route(None, None, ids_s, len(sample), cfg.E, cfg.k, "hash")
    else:
        lg = oracle.router_logits(xs, synth.router_weight(cfg))
        idx_s, _ = oracle.route(lg, synth.router_bias(cfg), None, len(sample), cfg.E, cfg.k,
                                cfg.route)
    experts = {int(e): synth.expert_matrices(cfg, int(e)) for e in np.unique(idx_s)}
    y_ref, _, _, _ = _oracle_layer(cfg, xs, ids_s, experts)
    r = rel_l2(y[sample], y_ref)
    banner(f"cfg{cid} sampled rel_l2={r:.3e}")
    assert r <= 2e-3


def test_decode_sweep_bitwise_and_oracle():
    """Decode shape (recipe 4): T = 1..64 from one token pool; every row is
    bitwise equal to the same token's row at T = 64; a sample vs the oracle."""
    cfg = synth.CONFIGS[4]
    banner("decode sweep recipe 4")
    dl, layer = _device_layer(4)
    pool = synth.x_tokens(cfg)  # 64 tokens
    y64 = to_np(layer.forward(dev(pool)))
    for T in range(1, 65):
        y = to_np(layer.forward(dev(np.ascontiguousarray(pool[:T]))))
        assert np.array_equal(y, y64[:T]), T
    rng = np.random.default_rng(4)
    for _ in range(3):
        perm = rng.permutation(64)[:17]
        y = to_np(layer.forward(dev(np.ascontiguousarray(pool[perm]))))
        assert np.array_equal(y, y64[perm])
    sample = np.array([0, 31, 63])
    xs = np.ascontiguousarray(pool[sample])
    lg = oracle.router_logits(xs, synth.router_weight(cfg))
    idx_s, _ = oracle.route(lg, synth.router_bias(cfg), None, 3, cfg.E, cfg.k, cfg.route)
    experts = {int(e): synth.expert_matrices(cfg, int(e)) for e in np.unique(idx_s)}
    y_ref, _, _, _ = _oracle_layer(cfg, xs, None, experts)
    assert rel_l2(y64[sample], y_ref) <= 2e-3


def test_prefill_rows_equal_decode_rows():
    """Tokens of the 4096-token prefill batch give the same bits when run alone
    (different GEMM tile shapes, same MFMA chain)."""
    cfg = synth.CONFIGS[3]
    banner("prefill vs decode rows recipe 3")
    dl, layer = _device_layer(3)
    x = synth.x_tokens(cfg)
    y = to_np(layer.forward(dev(x)))
    for sel in ([0], [4095], [5, 77, 1000, 4000], list(range(100, 164))):
        ys = to_np(layer.forward(dev(np.ascontiguousarray(x[sel]))))
        assert np.array_equal(ys, y[sel]), sel


def test_edge_cases():
    banner("edge cases")
    cfg = synth.CONFIGS[2]
    dl, layer = _device_layer(2)
    x = synth.x_tokens(cfg, T=3)
    # T = 0 is a no-op
    y0 = layer.forward(dev(np.zeros((0, cfg.D), np.uint16)))
    assert y0.shape == (0, cfg.D)
    # all tokens to the same experts through a huge bias
    big = torch.zeros(cfg.E, device="cuda")
    big[[5, 6, 7, 8, 9, 10]] = 1000.0
    l2 = moe.MoELayer(dl.w_router, big, layer.routed, layer.shared, cfg.E, cfg.k, "sigmoid")
    xx = synth.x_tokens(cfg, T=130)
    y = to_np(l2.forward(dev(xx)))
    bias_np = big.cpu().numpy()
    experts = {e: synth.expert_matrices(cfg, e) for e in range(5, 11)}
    y_ref, idx_ref, _, _ = oracle.layer_forward(xx, None, synth.router_weight(cfg), bias_np,
                                                experts, synth.shared_matrices(cfg), 130, cfg.D,
                                                cfg.E, cfg.k, cfg.I, cfg.I_shared, "sigmoid",
                                                "bf16")
    assert set(np.unique(idx_ref)) == set(range(5, 11))
    assert rel_l2(y, y_ref) <= 2e-3
    # k = 1, no shared expert, softmax
    l3 = moe.MoELayer(dl.w_router, None, layer.routed, None, cfg.E, 1, "softmax")
    y = to_np(l3.forward(dev(x)))
    experts = {e: synth.expert_matrices(cfg, e) for e in range(cfg.E)}
    y_ref, _, _, _ = oracle.layer_forward(x, None, synth.router_weight(cfg), None, experts, None,
                                          3, cfg.D, cfg.E, 1, cfg.I, 0, "softmax", "bf16")
    assert rel_l2(y, y_ref) <= 2e-3
