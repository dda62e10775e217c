"""Helpers shared by the GPU tests (comparison and conversions only)."""
import numpy as np
import pytest
import torch

import oracle

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    g, r = as_f64(got), as_f64(ref)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g - r))


def tol_for(act: str) -> float:
    """Output tolerance (relative L2 over the whole output, in fp64)."""
    return 1e-5 if act == "f32" else 2e-3


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def banner(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)


def mxfp4_decode_bf16(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Oracle decode of MXFP4 codes/scales [G, rows, cols/2], [G, rows, cols/32] to
    bf16 bit patterns [G, rows, cols]."""
    G, rows, half = packed.shape
    lo, hi = packed & 0xF, packed >> 4
    codes = np.stack([lo, hi], -1).reshape(G, rows, half * 2)
    sc = np.repeat(scales, 32, axis=-1)
    table = np.array([[oracle.lib().orc_mxfp4_value(c, s) for s in range(256)] for c in range(16)])
    return oracle.bf16_from_f64_array(table[codes, sc])


def mxfp4_pack(codes: np.ndarray) -> np.ndarray:
    """E2M1 codes [..., cols] -> bytes [..., cols/2], element 2i in the low nibble."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


_layers = {}


def device_layer(cid):
    """(DeviceLayer, MoELayer) of a recipe, uploaded once; one large layer is
    kept resident at a time (recipe 4 shares recipe 3's weights)."""
    import synth
    from synth import device as sdev
    if cid == 4:  # the decode recipe runs the prefill recipe's layer
        cid = 3
    if cid not in _layers:
        _layers.clear()
        cfg = synth.CONFIGS[cid]
        dl = sdev.upload_layer(cfg, "cuda",
                               progress=lambda e, n: banner(f"recipe {cid}: {e}/{n} experts"))
        _layers[cid] = (dl, sdev.layer_object(dl))
    return _layers[cid]
