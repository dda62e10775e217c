"""Upload of the seeded synthetic layer inputs to a GPU (torch tensors).

Only copies bytes produced by this package's generator; no arithmetic of the
layer.  Expert weights are generated expert by expert on the host and copied
into one preallocated device tensor, so a 22 GB weight set never needs a
second host copy.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import synth


def _to_dev(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return _to_dev(bits, device)


def tensor_to_numpy(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclass
class DeviceLayer:
    cfg: synth.LayerConfig
    w_router: Optional[torch.Tensor]
    bias: Optional[torch.Tensor]
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    gate_scale: Optional[torch.Tensor]
    up_scale: Optional[torch.Tensor]
    down_scale: Optional[torch.Tensor]
    sh_gate: Optional[torch.Tensor]
    sh_up: Optional[torch.Tensor]
    sh_down: Optional[torch.Tensor]
    host_experts: Optional[dict] = None  # expert id -> host matrices kept by upload_layer


def upload_layer(cfg: synth.LayerConfig, device="cuda", keep_experts=(),
                 progress=None) -> DeviceLayer:
    """Generates the layer's weights expert by expert and copies them to the
    device; the host matrices of the experts in keep_experts are kept (for a
    CPU computation on the same bytes without generating them again).
    progress(e, E), if given, is called every 64 experts."""
    E, I, D = cfg.E, cfg.I, cfg.D
    mx = cfg.wdtype == "mxfp4"
    if mx:
        tdt = torch.uint8
        gate = torch.empty((E, I, D // 2), dtype=tdt, device=device)
        up = torch.empty_like(gate)
        down = torch.empty((E, D, I // 2), dtype=tdt, device=device)
        gs = torch.empty((E, I, D // 32), dtype=tdt, device=device)
        us = torch.empty_like(gs)
        ds = torch.empty((E, D, I // 32), dtype=tdt, device=device)
    else:
        tdt = torch.float32 if cfg.wdtype == "f32" else torch.bfloat16
        gate = torch.empty((E, I, D), dtype=tdt, device=device)
        up = torch.empty_like(gate)
        down = torch.empty((E, D, I), dtype=tdt, device=device)
        gs = us = ds = None
    kept = {}
    for e in range(E):
        if progress is not None and e % 64 == 0 and e:
            progress(e, E)
        g, u, d = synth.expert_matrices(cfg, e)
        if e in keep_experts:
            kept[e] = (g, u, d)
        if mx:
            gate[e].copy_(torch.from_numpy(g[0]))
            gs[e].copy_(torch.from_numpy(g[1]))
            up[e].copy_(torch.from_numpy(u[0]))
            us[e].copy_(torch.from_numpy(u[1]))
            down[e].copy_(torch.from_numpy(d[0]))
            ds[e].copy_(torch.from_numpy(d[1]))
        else:
            gate[e].copy_(_to_dev(g, "cpu"))
            up[e].copy_(_to_dev(u, "cpu"))
            down[e].copy_(_to_dev(d, "cpu"))
    sh = synth.shared_matrices(cfg)
    shg = shu = shd = None
    if sh is not None:
        shg, shu, shd = (_to_dev(m, device).unsqueeze(0).contiguous() for m in sh)
    wr = bias = None
    if cfg.route != "hash":
        wr = _to_dev(synth.router_weight(cfg), device)
        b = synth.router_bias(cfg)
        bias = None if b is None else torch.from_numpy(b).to(device)
    return DeviceLayer(cfg, wr, bias, gate, up, down, gs, us, ds, shg, shu, shd, kept)


def layer_object(dl: DeviceLayer, glu: str = "swiglu", w4a8: bool = False):
    """The binding's MoELayer over uploaded weights (glu: the experts' gated activation;
    w4a8: MXFP4 routed experts on MXFP8 activations)."""
    import invariant_moe_amd as moe
    routed = moe.ExpertWeights(dl.gate, dl.up, dl.down, dl.gate_scale, dl.up_scale, dl.down_scale)
    shared = None
    if dl.sh_gate is not None:
        shared = moe.ExpertWeights(dl.sh_gate, dl.sh_up, dl.sh_down)
    return moe.MoELayer(dl.w_router, dl.bias, routed, shared, dl.cfg.E, dl.cfg.k, dl.cfg.route,
                        glu=glu, w4a8=w4a8)


def x_device(cfg: synth.LayerConfig, device="cuda", T=None, offset_tokens=0) -> torch.Tensor:
    return _to_dev(synth.x_tokens(cfg, T=T, offset_tokens=offset_tokens), device)


def token_ids_device(cfg: synth.LayerConfig, device="cuda", T=None, offset_tokens=0):
    if cfg.route != "hash":
        return None
    return torch.from_numpy(synth.token_ids(cfg, T=T, offset_tokens=offset_tokens)).to(device)
