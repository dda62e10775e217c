"""moe_layer_forward_noalloc (the layer on the library's fixed device scratch,
for callers that cannot allocate) against moe_layer_forward with a caller
workspace: bit-identical outputs, on two calls in a row (the second with a
smaller batch, so it runs on the scratch the first one left behind), through
the C-ABI."""
import ctypes

import numpy as np
import pytest
import torch

import invariant_moe_amd as moe
import synth
from gpu_util import banner, dev, requires_gpu, to_np
from synth import device as sdev

pytestmark = [pytest.mark.gpu, requires_gpu]


def _noalloc(L, x, ids, dl, routed, shared, cfg, flags, y, stream):
    T, D = x.shape
    r = routed.as_struct()
    s = shared.as_struct() if shared is not None else None
    return L.moe_layer_forward_noalloc(
        x.data_ptr(), None if ids is None else ids.data_ptr(),
        None if dl.w_router is None else dl.w_router.data_ptr(),
        None if dl.bias is None else dl.bias.data_ptr(), ctypes.byref(r),
        ctypes.byref(s) if s is not None else None, T, D, cfg.E, cfg.k, cfg.I,
        cfg.I_shared if shared is not None else 0, moe.ROUTE[cfg.route],
        moe.F32 if cfg.act == "f32" else moe.BF16, flags,
        y.data_ptr(), stream.cuda_stream)


@pytest.mark.parametrize("cid,Ts", [(2, (300, 37)), (2, (512, 1)), (1, (64, 5))])
def test_noalloc_equals_workspace_path(cid, Ts):
    cfg = synth.CONFIGS[cid]
    banner(f"noalloc recipe {cid} T={Ts}")
    dl = sdev.upload_layer(cfg, "cuda")
    routed = moe.ExpertWeights(dl.gate, dl.up, dl.down, dl.gate_scale, dl.up_scale,
                               dl.down_scale)
    shared = (moe.ExpertWeights(dl.sh_gate, dl.sh_up, dl.sh_down) if dl.sh_gate is not None
              else None)
    L = moe.lib()
    st = torch.cuda.current_stream()
    for T in Ts:
        c = cfg.with_T(T)
        x = sdev.x_device(c, "cuda")
        ids = sdev.token_ids_device(c, "cuda")
        ref = moe.layer_forward(x, ids, dl.w_router, dl.bias, routed, shared, cfg.E, cfg.k,
                                cfg.route)
        y = torch.full((T, cfg.D), float("nan"), dtype=x.dtype, device="cuda")
        rc = _noalloc(L, x, ids, dl, routed, shared, cfg, 0, y, st)
        assert rc == 0, L.moe_last_error()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(y), to_np(ref)), (cid, T)
    # the binding's wrapper, with the output passed in (nothing allocated)
    y2 = torch.empty_like(y)
    moe.layer_forward_noalloc(x, ids, dl.w_router, dl.bias, routed, shared, cfg.E, cfg.k,
                              cfg.route, out=y2)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(y2), to_np(ref))


def test_noalloc_rejects_layers_past_the_scratch():
    """A batch whose workspace exceeds MOE_NOALLOC_SCRATCH_BYTES is refused
    with MOE_ERR_WORKSPACE before anything is launched (output untouched)."""
    cfg = synth.CONFIGS[2]
    banner("noalloc size limit")
    L = moe.lib()
    T = 8192  # recipe-2 layer: about 130 MB of workspace
    need = L.moe_layer_workspace_bytes(T, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, moe.BF16,
                                       moe.BF16)
    assert need > moe.NOALLOC_SCRATCH_BYTES
    dl = sdev.upload_layer(cfg, "cuda")
    routed = moe.ExpertWeights(dl.gate, dl.up, dl.down)
    shared = moe.ExpertWeights(dl.sh_gate, dl.sh_up, dl.sh_down)
    x = torch.zeros((T, cfg.D), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, cfg.D), 3.0, dtype=torch.bfloat16, device="cuda")
    rc = _noalloc(L, x, None, dl, routed, shared, cfg, 0, y, torch.cuda.current_stream())
    assert rc == -5 and b"MOE_NOALLOC_SCRATCH_BYTES" in L.moe_last_error()
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
