"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function include/moe.h declares, and rejects bad arguments before
launching anything."""
import ctypes
import os
import re

import pytest

import invariant_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(moe.EXPORTS) <= set(names)
    assert L.moe_abi_version() == 3


def test_build_id_matches_sources():
    """The loaded binary carries the hash of the sources it was built from;
    it equals the hash of the checked-out sources (no stale binary)."""
    from invariant_moe_amd import _build
    got = moe.build_id()
    assert len(got) == 16 and int(got, 16) >= 0
    assert got == _build.source_hash()
    moe.check_build()


def test_status_strings():
    L = moe.lib()
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(-5) == b"MOE_ERR_WORKSPACE"


class _W(ctypes.Structure):
    _fields_ = moe._Weights._fields_


def _fake(addr=0x100000):
    return ctypes.c_void_p(addr)


def _weights(dtype=1, scales=False, addr=0x100000):
    w = moe._Weights(addr, addr + 4096, addr + 8192, None, None, None, dtype)
    if scales:
        w.gate_scale, w.up_scale, w.down_scale = addr + 16, addr + 32, addr + 48
    return w


def _layer(**kw):
    L = moe.lib()
    a = dict(x=_fake(), token_ids=None, w_router=_fake(), bias=None, routed=_weights(),
             shared=None, T=4, D=256, E=8, k=2, I=128, Is=0, mode=1, act=1, flags=0, y=_fake(),
             ws=_fake(), wsb=1 << 30, stream=None)
    a.update(kw)
    r = a["routed"]
    s = a["shared"]
    rc = L.moe_layer_forward(a["x"], a["token_ids"], a["w_router"], a["bias"],
                             ctypes.byref(r) if r is not None else None,
                             ctypes.byref(s) if s is not None else None, a["T"], a["D"], a["E"],
                             a["k"], a["I"], a["Is"], a["mode"], a["act"], a["flags"], a["y"],
                             a["ws"], a["wsb"], a["stream"])
    return rc, L.moe_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(routed=None), -1),
    (dict(x=None), -1),
    (dict(k=0), -2),
    (dict(k=9), -2),             # k > E
    (dict(k=33, E=64), -2),      # k above the 32 limit
    (dict(E=0), -2),
    (dict(E=1025, k=2), -2),
    (dict(T=-1), -2),
    (dict(D=100), -2),
    (dict(D=0), -2),
    (dict(I=48), -2),
    (dict(act=2), -3),           # MXFP4 activations
    (dict(routed=_weights(dtype=0)), -3),      # fp32 weights, bf16 acts
    (dict(routed=_weights(dtype=2)), -1),      # MXFP4 without scales
    (dict(routed=_weights(dtype=1, scales=True)), -3),
    (dict(x=_fake(0x100008)), -4),             # misaligned
    (dict(wsb=16), -5),
    (dict(ws=None), -5),
    (dict(flags=3), -6),         # both gated activations
    (dict(flags=8), -6),         # unknown flag bit
    (dict(flags=0x80000001), -6),
    (dict(mode=2), -1),          # hash without token ids
    (dict(mode=7), -2),
    (dict(shared=_weights(), Is=40), -2),
])
def test_layer_forward_rejects(kw, status):
    rc, msg = _layer(**kw)
    assert rc == status, (rc, msg)
    assert msg


def test_t_zero_is_a_noop_without_gpu_work():
    for flags in (0, 1, 2):  # every accepted gated activation
        rc, msg = _layer(T=0, flags=flags)
        assert rc == 0 and msg == ""


def test_workspace_query():
    L = moe.lib()
    small = L.moe_layer_workspace_bytes(64, 256, 8, 2, 128, 0, 0, 0)
    big = L.moe_layer_workspace_bytes(4096, 7168, 256, 8, 2048, 2048, 1, 1)
    assert 0 < small < big
    # h + o dominate: R*(I + D)*2 bytes at the DeepSeek-V3 prefill shape
    assert big >= 4096 * 8 * (2048 + 7168) * 2
    assert L.moe_router_workspace_bytes(10, 8, 2) == 0
    assert L.moe_permute_workspace_bytes(64, 8) >= 8 * 12


def test_other_entry_points_reject():
    L = moe.lib()
    w = _weights()
    for flags in (3, 4, 0x100):  # two activations / unknown bits
        assert L.moe_grouped_swiglu(_fake(), None, _fake(), 10, 4, 64, 64, ctypes.byref(w), 1,
                                    flags, _fake(), _fake(), 1 << 20, None) == -6
    assert L.moe_grouped_swiglu(_fake(), None, _fake(), 10, 4, 64, 40, ctypes.byref(w), 1, 0,
                                _fake(), _fake(), 1 << 20, None) == -2
    assert L.moe_combine(_fake(), _fake(), _fake(), _fake(), None, 4, 0, 64, 1, _fake(), None) == -2
    assert L.moe_permute(_fake(), 4, 2, 8, None, _fake(), _fake(), _fake(), None, 1, 64, None,
                         _fake(), 1 << 20, None) == -1
    assert L.moe_permute(_fake(), 4, 2, 8, _fake(), _fake(), _fake(), _fake(), None, 1, 64, None,
                         _fake(), 4, None) == -5
    assert L.moe_router_topk(_fake(), 1, _fake(), None, None, 4, 64, 8, 2, 2, _fake(), _fake(),
                             None, 0, None) == -1  # hash needs token ids
    assert L.moe_routing_scores(_fake(), 4, 2, _fake(), None) == -2


def test_norm_entry_points_reject():
    L = moe.lib()
    f = _fake()
    # moe_residual_rmsnorm(x, residual, gamma, eps, T, D, act, residual_out, normed, stream)
    assert L.moe_residual_rmsnorm(f, f, f, 1e-6, 0, 64, 1, f, f, None) == 0  # T = 0: no-op
    assert L.moe_residual_rmsnorm(f, f, f, 1e-6, 4, 48, 1, f, f, None) == -2  # D % 32
    assert L.moe_residual_rmsnorm(f, f, f, -1.0, 4, 64, 1, f, f, None) == -6  # eps < 0
    assert L.moe_residual_rmsnorm(f, f, f, float("inf"), 4, 64, 1, f, f, None) == -6
    assert L.moe_residual_rmsnorm(f, f, f, float("nan"), 4, 64, 1, f, f, None) == -6
    assert L.moe_residual_rmsnorm(f, None, f, 1e-6, 4, 64, 1, f, f, None) == -1
    assert L.moe_residual_rmsnorm(f, f, _fake(0x100008), 1e-6, 4, 64, 1, f, f, None) == -4
    assert L.moe_residual_rmsnorm(f, f, f, 1e-6, 4, 64, 2, f, f, None) == -3  # MXFP4 rows
    # moe_combine_rmsnorm(eo, idx, w, pair_row, shared, residual, gamma, eps, T, k, D, act, ro, n)
    assert L.moe_combine_rmsnorm(f, f, f, f, None, f, f, 1e-6, 4, 0, 64, 1, f, f, None) == -2
    assert L.moe_combine_rmsnorm(f, f, f, f, None, f, f, 1e-6, 4, 33, 64, 1, f, f, None) == -2
    assert L.moe_combine_rmsnorm(f, None, f, f, None, f, f, 1e-6, 4, 2, 64, 1, f, f, None) == -1
    assert L.moe_combine_rmsnorm(f, f, f, f, _fake(0x100004), f, f, 1e-6, 4, 2, 64, 1, f, f,
                                 None) == -4
    assert L.moe_combine_rmsnorm(f, f, f, f, None, f, f, -0.5, 4, 2, 64, 1, f, f, None) == -6


def test_w4a8_layer_flag_rejects():
    # bf16 routed weights, MXFP4 without multiples of 128, an MXFP4 shared expert
    assert _layer(flags=4)[0] == -3
    assert _layer(flags=4, routed=_weights(dtype=2, scales=True), D=288)[0] == -2
    assert _layer(flags=4, routed=_weights(dtype=2, scales=True), D=256, I=128,
                  shared=_weights(dtype=2, scales=True), Is=128)[0] == -6
    assert _layer(flags=8)[0] == -6  # unknown bit
    L = moe.lib()
    w = _weights()
    # the grouped entry points take no W4A8 bit; the W4A8 one needs MXFP4 weights
    assert L.moe_grouped_swiglu(_fake(), None, _fake(), 10, 4, 128, 128, ctypes.byref(w), 1, 4,
                                _fake(), _fake(), 1 << 20, None) == -6
    assert L.moe_grouped_swiglu_w4a8(_fake(), None, _fake(), 10, 4, 128, 128, ctypes.byref(w), 0,
                                      _fake(), _fake(), 1 << 20, None) == -3
    assert L.moe_grouped_swiglu_w4a8(_fake(), None, _fake(), 10, 4, 160, 128, ctypes.byref(w), 0,
                                      _fake(), _fake(), 1 << 20, None) == -2
    # the workspace query with MXFP4 weights covers the flag
    assert L.moe_layer_workspace_bytes(2048, 7168, 256, 8, 2048, 2048, 1, 2) > \
        L.moe_layer_workspace_bytes(2048, 7168, 256, 8, 2048, 2048, 1, 1)
