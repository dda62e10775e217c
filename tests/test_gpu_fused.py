"""The single-launch layer forward (moe_layer_forward_fused) on the GPU.

Its outputs must be bit-identical to the separate-kernel path
(moe_layer_forward), which the other GPU tests compare with the oracle, at
every batch size and routing mode; it is also checked against the oracle
directly.  After every call the task queue's header is back to zero and its
error word is clear (no wait gave up)."""
import numpy as np
import pytest
import torch

import invariant_moe_amd as moe
import oracle
import synth
from gpu_util import (banner, dev, device_layer, mxfp4_pack, rel_l2, requires_gpu, to_np)
from synth import device as sdev

pytestmark = [pytest.mark.gpu, requires_gpu]


def _fused(layer, x, ids, ws, glu="swiglu"):
    y = moe.layer_forward_fused(x, ids, layer.w_router, layer.bias, layer.routed, layer.shared,
                                layer.E, layer.k, layer.mode, workspace=ws, glu=glu)
    torch.cuda.synchronize()
    return y


def _header_clear(ws):
    p = (ws.data_ptr() + 255) // 256 * 256 - ws.data_ptr()
    return bool((ws[p:p + 256] == 0).all())


def _check_pair(layer, x, ids, ws, glu="swiglu"):
    ref = to_np(moe.layer_forward(x, ids, layer.w_router, layer.bias, layer.routed, layer.shared,
                                  layer.E, layer.k, layer.mode, glu=glu))
    got = to_np(_fused(layer, x, ids, ws, glu))
    assert moe.fused_error(ws) == 0
    assert _header_clear(ws)
    return got, ref


def test_fused_small_layer_every_T_bitwise():
    """Recipe 2 (T=512, D=1024, E=64+1, top-6 sigmoid): T = 1..64 and larger
    batches (every fused tile configuration), fused == unfused bit for bit;
    one workspace reused across all calls."""
    cfg = synth.CONFIGS[2]
    banner("fused recipe 2")
    dl, layer = device_layer(2)
    pool = synth.x_tokens(cfg)
    ws = moe.fused_workspace(cfg.T, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, "cuda")
    for T in list(range(1, 65)) + [100, 257, 512]:
        x = dev(np.ascontiguousarray(pool[:T]))
        got, ref = _check_pair(layer, x, None, ws)
        assert np.array_equal(got, ref), T


def test_fused_small_layer_vs_oracle():
    cfg = synth.CONFIGS[2]
    banner("fused recipe 2 vs oracle")
    dl, layer = device_layer(2)
    x = synth.x_tokens(cfg)
    ws = moe.fused_workspace(cfg.T, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, "cuda")
    y = to_np(_fused(layer, dev(x), None, ws))
    experts = {e: synth.expert_matrices(cfg, e) for e in range(cfg.E)}
    y_ref, _, _, _ = oracle.layer_forward(x, None, synth.router_weight(cfg),
                                          synth.router_bias(cfg), experts,
                                          synth.shared_matrices(cfg), cfg.T, cfg.D, cfg.E, cfg.k,
                                          cfg.I, cfg.I_shared, cfg.route, cfg.wdtype)
    r = rel_l2(y, y_ref)
    banner(f"fused recipe 2 rel_l2={r:.3e}")
    assert r <= 2e-3
    assert moe.fused_error(ws) == 0


@pytest.mark.parametrize("glu", ["clamp", "situ"])
def test_fused_glu_variants_and_softmax_bitwise(glu):
    """Gated-activation flags, softmax routing without a shared expert, k = 1."""
    cfg = synth.CONFIGS[2]
    banner(f"fused variants {glu}")
    dl, layer = device_layer(2)
    x = dev(synth.x_tokens(cfg, T=77))
    ws = moe.fused_workspace(77, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, "cuda")
    got, ref = _check_pair(layer, x, None, ws, glu)
    assert np.array_equal(got, ref)
    for k, shared in ((cfg.k, None), (1, layer.shared)):
        l2 = moe.MoELayer(dl.w_router, None, layer.routed, shared, cfg.E, k, "softmax")
        ws2 = moe.fused_workspace(77, cfg.D, cfg.E, k, cfg.I, cfg.I_shared, "cuda")
        got, ref = _check_pair(l2, x, None, ws2)
        assert np.array_equal(got, ref), k


def test_fused_moe_layer_option_and_streams():
    """MoELayer(fused=True) on the current stream and on a side stream."""
    cfg = synth.CONFIGS[2]
    banner("fused MoELayer option")
    dl, layer = device_layer(2)
    fl = sdev.layer_object(dl)
    fl.fused = True
    x = dev(synth.x_tokens(cfg, T=300))
    ref = to_np(layer.forward(x))
    assert np.array_equal(to_np(fl.forward(x)), ref)
    s = torch.cuda.Stream()
    y = fl.forward(x, stream=s)
    s.synchronize()
    assert np.array_equal(to_np(y), ref)


def _small_mxfp4_hash_layer():
    """A small hash-routed layer with MXFP4 routed experts and a bf16 shared
    expert (K % 64 == 32 in both GEMMs: D = 288, I = 96)."""
    E, D, I, IS = 8, 288, 96, 64
    rng = np.random.default_rng(7)

    def fp4(shape, lo, hi):
        codes = rng.integers(0, 16, size=shape, dtype=np.uint8)
        sc = rng.integers(lo, hi + 1, size=(shape[0], shape[1], shape[2] // 32), dtype=np.uint8)
        return dev(mxfp4_pack(codes)), dev(sc)

    g, u, d = fp4((E, I, D), 118, 121), fp4((E, I, D), 118, 121), fp4((E, D, I), 116, 119)
    routed = moe.ExpertWeights(g[0], u[0], d[0], g[1], u[1], d[1])
    sh = [synth.normal_bf16(71, t, n, 0.05) for t, n in ((0, IS * D), (1, IS * D), (2, D * IS))]
    shared = moe.ExpertWeights(dev(sh[0].reshape(1, IS, D)), dev(sh[1].reshape(1, IS, D)),
                               dev(sh[2].reshape(1, D, IS)))
    return moe.MoELayer(None, None, routed, shared, E, 3, "hash"), D


def test_fused_mxfp4_hash_bitwise():
    banner("fused MXFP4 + hash")
    layer, D = _small_mxfp4_hash_layer()
    for T in (1, 5, 40, 300, 1000):
        x = dev(synth.normal_bf16(72, 0, T * D, 1.0).reshape(T, D))
        ids = torch.from_numpy(synth.u32(72, 1, T).astype(np.int64) % 131072).to(
            torch.int32).cuda()
        ws = moe.fused_workspace(T, D, layer.E, layer.k, 96, 64, "cuda")
        got, ref = _check_pair(layer, x, ids, ws)
        assert np.array_equal(got, ref), T


def test_fused_edge_cases():
    cfg = synth.CONFIGS[2]
    banner("fused edges")
    dl, layer = device_layer(2)
    ws = moe.fused_workspace(4, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, "cuda")
    y0 = moe.layer_forward_fused(dev(np.zeros((0, cfg.D), np.uint16)), None, layer.w_router,
                                 layer.bias, layer.routed, layer.shared, cfg.E, cfg.k, "sigmoid",
                                 workspace=ws)
    assert y0.shape == (0, cfg.D)
    # every token to the same six experts (one expert group holds all rows)
    big = torch.zeros(cfg.E, device="cuda")
    big[[5, 6, 7, 8, 9, 10]] = 1000.0
    l2 = moe.MoELayer(dl.w_router, big, layer.routed, layer.shared, cfg.E, cfg.k, "sigmoid")
    x = dev(synth.x_tokens(cfg, T=130))
    ws2 = moe.fused_workspace(130, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, "cuda")
    got, ref = _check_pair(l2, x, None, ws2)
    assert np.array_equal(got, ref)
    # fp32 activations and the FP4 x FP8 flag are refused before any launch
    with pytest.raises(moe.MoEError):
        moe.layer_forward_fused(torch.zeros((2, cfg.D), device="cuda"), None,
                                layer.w_router.float(), None, layer.routed, None, cfg.E, cfg.k,
                                "sigmoid", workspace=ws)


def test_fused_decode_sweep_bitwise():
    """The DeepSeek-V3-shaped layer at decode batch sizes T = 1..64 (recipe 4
    pool): fused == unfused for every T."""
    cfg = synth.CONFIGS[4]
    banner("fused decode sweep")
    dl, layer = device_layer(4)
    pool = synth.x_tokens(cfg)
    ws = moe.fused_workspace(64, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, "cuda")
    for T in range(1, 65):
        x = dev(np.ascontiguousarray(pool[:T]))
        got, ref = _check_pair(layer, x, None, ws)
        assert np.array_equal(got, ref), T


def test_fused_prefill_bitwise():
    """The DeepSeek-V3-shaped prefill batch (T = 4096): fused == unfused over
    the whole output."""
    cfg = synth.CONFIGS[3]
    banner("fused prefill recipe 3")
    dl, layer = device_layer(3)
    x = dev(synth.x_tokens(cfg))
    ws = moe.fused_workspace(cfg.T, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, "cuda")
    got, ref = _check_pair(layer, x, None, ws)
    assert np.array_equal(got, ref)
